// Host-side checks of the cache index helpers and of the launch plans the
// C ABI makes, meant to be built with AddressSanitizer and
// UndefinedBehaviorSanitizer.  No GPU is used: the kernel launchers that
// plan.cpp calls are replaced below by recorders, so every compute entry
// point runs its argument checks and planning and hands its launch
// arguments here instead of to the device.  Device pointers are stand-ins
// that are never dereferenced.
//
// Checked:
//   - decode_split_range: the splits of a sequence cover its visible key
//     blocks exactly once, in order, and their key ranges partition the
//     visible keys;
//   - k_elem_offset / v_elem_offset: bijections from (slot, dim) onto the
//     elements of a segment, K rows 16 contiguous bytes per 8 dims;
//   - clamp_page: results inside [0, n_pages);
//   - decode plans: for every sequence length up to the call's bound, the
//     grid holds every split the kernels will compute, merges stay within
//     their size class, and every partial-result and counter index lies in
//     the bound workspace;
//   - prefill plans: the row blocks cover the chunk's (token, head) rows.
//
// Prints "host_check OK" and exits 0, or lists the failures and exits 1.

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <vector>

#include "../../decode_attention_gemma_amd/csrc/internal.h"
#include "../../include/g4attn.h"

namespace {

int g_failures = 0;

#define CHECK(cond, ...)                                 \
  do {                                                   \
    if (!(cond)) {                                       \
      if (++g_failures <= 40) {                          \
        std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
        std::printf(__VA_ARGS__);                        \
        std::printf("\n");                               \
      }                                                  \
    }                                                    \
  } while (0)

// ---- recorders standing in for the kernel launchers ----------------------

struct DecodeCall {
  g4::DecodeArgs a;
  int head_dim, batch;
  bool k_eq_v;
};
std::vector<DecodeCall> g_decode;
std::vector<g4::MergeArgs> g_merge;
std::vector<g4::PrefillArgs> g_prefill;
std::vector<std::pair<g4::AppendArgs, int>> g_append;
alignas(256) unsigned char g_fake_scratch[256];

}  // namespace

namespace g4 {
hipError_t launch_append(const AppendArgs& a, int batch, hipStream_t) {
  g_append.push_back({a, batch});
  return hipSuccess;
}
hipError_t launch_decode(int head_dim, bool k_eq_v, const DecodeArgs& a, int batch, hipStream_t) {
  g_decode.push_back({a, head_dim, batch, k_eq_v});
  return hipSuccess;
}
hipError_t launch_prefill(int, bool, const PrefillArgs& a, hipStream_t) {
  g_prefill.push_back(a);
  return hipSuccess;
}
hipError_t launch_merge(const MergeArgs& a, hipStream_t) {
  g_merge.push_back(a);
  return hipSuccess;
}
hipError_t scratch_address(void** ptr, bool* first_use) {
  *ptr = g_fake_scratch;  // stands for the device array; never dereferenced here
  *first_use = false;
  return hipSuccess;
}
hipError_t launch_zero(int32_t*, int, hipStream_t) { return hipSuccess; }
}  // namespace g4

const char* hipGetErrorString(hipError_t) { return "(launch recorder)"; }

namespace {

// ---- index helpers --------------------------------------------------------

void check_split_ranges() {
  std::mt19937 rng(7);
  auto one = [&](int lo, int L, int KB, int bps) {
    int n_used = -1, f = 0, e = 0;
    g4::decode_split_range(lo, L, KB, bps, 0, &n_used, &f, &e);
    const int nb = L > lo ? (L + KB - 1) / KB - lo / KB : 0;
    CHECK(n_used == (nb + bps - 1) / bps, "n_used %d for nb %d bps %d", n_used, nb, bps);
    int next_blk = lo / KB;
    int next_key = lo;
    for (int s = 0; s < n_used + 2; ++s) {
      int nu = 0;
      g4::decode_split_range(lo, L, KB, bps, s, &nu, &f, &e);
      CHECK(nu == n_used, "n_used differs between splits");
      if (s >= n_used) {
        CHECK(f == e, "split %d past n_used %d is not empty", s, n_used);
        continue;
      }
      CHECK(f == next_blk && e > f && e - f <= bps,
            "lo %d L %d KB %d bps %d split %d: blocks [%d, %d), expected start %d", lo, L, KB,
            bps, s, f, e, next_blk);
      next_blk = e;
      const int r_beg = std::max(lo, f * KB), r_end = std::min(L, e * KB);
      CHECK(r_beg == next_key && r_end > r_beg, "split %d keys [%d, %d), expected start %d", s,
            r_beg, r_end, next_key);
      next_key = r_end;
    }
    CHECK(next_blk == lo / KB + nb, "blocks end at %d, expected %d", next_blk, lo / KB + nb);
    CHECK(next_key == std::max(lo, L), "keys end at %d, expected %d", next_key, std::max(lo, L));
  };
  for (int KB : {16, 32})
    for (int W : {0, 1, 8, 512, 1024})
      for (int L = 0; L <= 2200; L += (L < 80 ? 1 : 37))
        for (int bps : {1, 2, 3, 4, 7, 8, 16, 17, 33, 257}) one(W > 0 ? std::max(0, L - W) : 0, L, KB, bps);
  for (int i = 0; i < 20000; ++i) {
    const int L = (int)(rng() % 70000);
    const int W = (int)(rng() % 3) == 0 ? 0 : 1 + (int)(rng() % 4096);
    one(W > 0 ? std::max(0, L - W) : 0, L, (rng() & 1) ? 16 : 32, 1 + (int)(rng() % 300));
  }
}

void check_elem_offsets() {
  for (int D : {32, 64, 128, 256, 512})
    for (int cap : {64, 128, 1088}) {
      const int64_t n = (int64_t)cap * D;
      std::vector<unsigned char> seen_k(n, 0), seen_v(n, 0);
      for (int slot = 0; slot < cap; ++slot)
        for (int d = 0; d < D; ++d) {
          const int64_t ok = g4::k_elem_offset(slot, d, D), ov = g4::v_elem_offset(slot, d, D);
          CHECK(ok % 2 == 0 && ov % 2 == 0, "odd byte offset");
          CHECK(ok >= 0 && ok / 2 < n && ov >= 0 && ov / 2 < n,
                "D %d cap %d (slot %d, d %d) outside the segment", D, cap, slot, d);
          if (ok >= 0 && ok / 2 < n) ++seen_k[ok / 2];
          if (ov >= 0 && ov / 2 < n) ++seen_v[ov / 2];
          if (d % 8 != 7)
            CHECK(g4::k_elem_offset(slot, d + 1, D) == ok + 2, "K row chunk not contiguous");
        }
      for (int64_t i = 0; i < n; ++i) {
        CHECK(seen_k[i] == 1, "D %d cap %d: K element %lld hit %d times", D, cap, (long long)i,
              (int)seen_k[i]);
        CHECK(seen_v[i] == 1, "D %d cap %d: V element %lld hit %d times", D, cap, (long long)i,
              (int)seen_v[i]);
        if (seen_k[i] != 1 || seen_v[i] != 1) return;
      }
    }
}

void check_clamp_page() {
  for (int n_pages : {1, 2, 7, 1000})
    for (int id = -5; id < n_pages + 5; ++id) {
      const int c = g4::clamp_page(id, n_pages);
      CHECK(c >= 0 && c < n_pages, "clamp_page(%d, %d) = %d", id, n_pages, c);
      if (id >= 0 && id < n_pages) CHECK(c == id, "clamp_page moved an in-range id");
    }
}

// ---- plans through the C ABI ----------------------------------------------

g4attn_layer_desc desc(int nq, int nkv, int d, int window, int keqv, int owner = -1) {
  g4attn_layer_desc x{};
  x.n_q_heads = nq;
  x.n_kv_heads = nkv;
  x.head_dim = d;
  x.window = window;
  x.k_eq_v = keqv;
  x.kv_owner_layer = owner;
  x.scale = 0.0625f;
  x.softcap = 0.f;
  return x;
}

constexpr size_t kFakeBase = size_t(1) << 40;  // stand-in device addresses

// Every decode launch recorded so far: grid coverage, merge class, and
// workspace bounds, for each sequence length the kernels may see.
void check_decode_calls(const g4attn_stack* st, const std::vector<g4attn_layer_desc>& layers,
                        int layer, uint64_t ws_bytes, const char* what) {
  const g4attn_layer_desc& d = layers[layer];
  for (const DecodeCall& c : g_decode) {
    const g4::DecodeArgs& a = c.a;
    const int KB = g4::kDecodeBlock;
    const int nh = std::min(16, a.G);
    CHECK(a.n_splits >= 1 && a.n_splits <= g4::kMaxDecodeSplits, "%s: n_splits %d", what,
          a.n_splits);
    CHECK(a.G * a.n_kv == a.n_q && a.n_q == d.n_q_heads, "%s: head counts", what);
    CHECK(a.n_hblk == (a.G + 15) / 16, "%s: head blocks", what);
    for (int L = 0; L <= a.max_len; L += (L < 300 ? 1 : 13)) {
      const int lo = a.window > 0 ? std::max(0, L - a.window) : 0;
      int n_used, f, e;
      g4::decode_split_range(lo, L, KB, a.blocks_per_split, 0, &n_used, &f, &e);
      CHECK(n_used <= a.n_splits, "%s: L %d needs %d splits, grid has %d", what, L, n_used,
            a.n_splits);
      if (n_used > a.n_splits) break;
    }
    if (a.merge_in_kernel)
      CHECK((int64_t)a.n_splits * nh * c.head_dim * 4 <= 64 * 1024 && a.n_splits <= 8,
            "%s: in-kernel merge of %d splits", what, a.n_splits);
    // workspace: counters, (m, l) and partials of every (row, split) slot
    const uint64_t base = kFakeBase + (1 << 20);
    const uint64_t ctr_end = (uint64_t)(uintptr_t)a.counters - base +
                             (uint64_t)c.batch * a.n_kv * a.n_hblk * 4;
    const uint64_t slots = (uint64_t)c.batch * a.n_q * a.n_splits;
    const uint64_t ml_beg = (uint64_t)(uintptr_t)a.part_ml - base;
    const uint64_t o_beg = (uint64_t)(uintptr_t)a.part_o - base;
    CHECK((uint64_t)(uintptr_t)a.counters >= base && ctr_end <= ml_beg, "%s: counters overlap",
          what);
    CHECK(ml_beg + slots * 8 <= o_beg, "%s: (m, l) slots overlap the partials", what);
    CHECK(o_beg + slots * c.head_dim * 4 <= ws_bytes, "%s: partials end at %llu > %llu", what,
          (unsigned long long)(o_beg + slots * c.head_dim * 4), (unsigned long long)ws_bytes);
  }
  (void)st;
}

void check_plans() {
  // 12B-shaped stack (sliding 16q/8kv D256 W1024; global 16q/1kv D512 k_eq_v)
  // and one with KV-shared layers and small heads
  std::vector<g4attn_layer_desc> layers = {desc(16, 8, 256, 1024, 0), desc(16, 1, 512, 0, 1),
                                           desc(8, 2, 256, 512, 0), desc(4, 1, 64, 0, 1),
                                           desc(8, 2, 256, 512, 0, 2), desc(32, 2, 128, 0, 0)};
  for (int max_batch : {1, 16, 64, 300}) {
    g4attn_stack* st = nullptr;
    CHECK(g4attn_stack_create(layers.data(), (int)layers.size(), max_batch, 32768, 64, &st) ==
              G4ATTN_OK, "create: %s", g4attn_last_error());
    if (!st) continue;
    uint64_t ws = 0, cb = 0;
    g4attn_workspace_bytes(st, &ws);
    g4attn_cache_bytes(st, &cb);
    void* cache = reinterpret_cast<void*>(kFakeBase);
    void* wsp = reinterpret_cast<void*>(kFakeBase + (1 << 20));
    CHECK(g4attn_bind(st, cache, wsp) == G4ATTN_OK, "bind: %s", g4attn_last_error());
    void* dev = reinterpret_cast<void*>(kFakeBase + (size_t(1) << 38));
    const int32_t* lens = reinterpret_cast<const int32_t*>(dev);
    for (int layer = 0; layer < (int)layers.size(); ++layer)
      for (int batch : {1, 2, 7, 16, 64, 300}) {
        if (batch > max_batch) continue;
        for (int max_len : {1, 17, 511, 1024, 1025, 4096, 32768}) {
          g_decode.clear();
          char what[96];
          std::snprintf(what, sizeof what, "layer %d batch %d max_len %d", layer, batch, max_len);
          const int rc = g4attn_decode(st, layer, dev, lens, batch, max_len, dev, nullptr);
          CHECK(rc == G4ATTN_OK, "%s: decode rc %d (%s)", what, rc, g4attn_last_error());
          CHECK(g_decode.size() == 1, "%s: %zu decode launches", what, g_decode.size());
          check_decode_calls(st, layers, layer, ws, what);
          g_decode.clear();
          const int rc2 = g4attn_decode_noalloc(st, layer, dev, lens, batch, max_len, dev, nullptr);
          CHECK(rc2 == G4ATTN_OK || rc2 == G4ATTN_ERR_UNSUPPORTED, "%s: noalloc rc %d", what, rc2);
        }
      }
    // prefill: row blocks cover T * G rows; the grid covers every row block
    for (int layer = 0; layer < (int)layers.size(); ++layer)
      for (int T : {1, 5, 64}) {
        g_prefill.clear();
        const int batch = std::min(max_batch, 4);
        const int rc = g4attn_prefill(st, layer, dev, lens, batch, T, 4032, dev, nullptr);
        CHECK(rc == G4ATTN_OK, "prefill rc %d (%s)", rc, g4attn_last_error());
        for (const g4::PrefillArgs& a : g_prefill) {
          CHECK(a.rows == T * a.G, "prefill rows %d for T %d G %d", a.rows, T, a.G);
          CHECK(a.n_rowblk * g4::kPrefillRows >= a.rows &&
                    (a.n_rowblk - 1) * g4::kPrefillRows < a.rows,
                "prefill row blocks %d for %d rows", a.n_rowblk, a.rows);
        }
      }
    // rejections stay rejections (and touch nothing)
    CHECK(g4attn_decode(st, 0, dev, lens, max_batch + 1, 10, dev, nullptr) == G4ATTN_ERR_RANGE,
          "batch beyond max_batch accepted");
    CHECK(g4attn_decode(st, 0, dev, lens, 1, 32769, dev, nullptr) == G4ATTN_ERR_RANGE,
          "max_seq_len beyond kv_max accepted");
    CHECK(g4attn_decode(st, 99, dev, lens, 1, 10, dev, nullptr) == G4ATTN_ERR_RANGE,
          "bad layer accepted");
    // key ranges and cache offsets against their definitions
    for (int layer = 0; layer < (int)layers.size(); ++layer) {
      const int W = layers[layer].window;
      for (int64_t qp : {0, 1, 7, 511, 1023, 1024, 5000})
        for (int64_t nk : {0, 1, 8, 1024, 6000}) {
          int64_t lo = -1, hi = -1;
          g4attn_key_range(st, layer, qp, nk, &lo, &hi);
          const int64_t h = std::max<int64_t>(0, std::min(qp + 1, nk));
          const int64_t l = std::min(h, W > 0 ? std::max<int64_t>(0, qp - W + 1) : 0);
          CHECK(lo == l && hi == h, "key_range layer %d q %lld n %lld: [%lld, %lld)", layer,
                (long long)qp, (long long)nk, (long long)lo, (long long)hi);
        }
      int32_t cap = 0;
      g4attn_layer_capacity(st, layer, &cap);
      CHECK(cap % 64 == 0 && cap > 0, "capacity %d", cap);
      const int D = layers[layer].head_dim;
      std::set<int64_t> seen;
      for (int64_t pos = 0; pos < cap; pos += (cap > 2048 ? 61 : 1))
        for (int dd = 0; dd < D; dd += 7) {
          int64_t ok = -1, ov = -1;
          CHECK(g4attn_kv_offset(st, layer, max_batch - 1, layers[layer].n_kv_heads - 1, pos, dd,
                                 &ok, &ov) == G4ATTN_OK, "kv_offset rejected");
          CHECK(ok >= 0 && (uint64_t)ok + 2 <= cb && ov >= 0 && (uint64_t)ov + 2 <= cb,
                "kv_offset outside the cache");
          CHECK(seen.insert(ok).second, "kv_offset repeats a K element");
        }
    }
    g4attn_stack_destroy(st);
  }
}

}  // namespace

int main() {
  check_split_ranges();
  check_elem_offsets();
  check_clamp_page();
  check_plans();
  if (g_failures) {
    std::printf("host_check: %d failure(s)\n", g_failures);
    return 1;
  }
  std::printf("host_check OK\n");
  return 0;
}
