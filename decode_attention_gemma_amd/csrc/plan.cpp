// Host side of the g4attn C ABI: descriptor validation, owner resolution,
// cache / workspace planning, the bit-exact index hooks, and argument checks
// before every kernel launch.  Nothing here allocates device memory.
//
// Owner rules follow "Porting Gemma-4 (2B / 4B / 12B) to AWS Inferentia2",
// 2.1 (a KV-shared layer attends to an earlier layer's K/V and holds no cache;
// only owning layers allocate one).  The resident cache of fixed capacity
// follows section 5 of the same page.

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/g4attn.h"
#include "internal.h"

struct LayerPlan {
  g4attn_layer_desc d;
  int owner;
  int cap;          // slots per (sequence, KV head) of the owner's planes
  uint64_t k_off;   // byte offset of the owner's K plane in the cache
  uint64_t v_off;   // byte offset of the owner's V plane (== k_off when k_eq_v)
};

struct g4attn_stack {
  std::vector<LayerPlan> L;
  int max_batch = 0, kv_max = 0, max_chunk = 0;
  // paged cache: pages of `page` slots, n_pages per plane, kv_max / page
  // block-table entries per sequence
  int paged = 0, page = 0, n_pages = 0;
  uint64_t cache_bytes = 0;
  uint64_t ws_ctr_off = 0, ws_ml_off = 0, ws_o_off = 0, ws_bytes = 0;
  uint64_t ctr_count = 0, ml_floats = 0, o_floats = 0;
  char* cache = nullptr;
  char* ws = nullptr;
};

namespace {

thread_local std::string g_err;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int32_t ok() {
  g_err.clear();
  return G4ATTN_OK;
}

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

bool head_dim_supported(int d) { return d == 32 || d == 64 || d == 128 || d == 256 || d == 512; }

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Slots per (sequence, KV head): always a multiple of 64 so that the 16- and
// 32-slot operand blocks never straddle the ring's wrap.  Global layers keep
// every position (kv_max rounded up); sliding layers keep a ring that holds a
// window plus one chunk of new tokens, so its size does not grow with context.
int layer_cap(const g4attn_layer_desc& d, int kv_max, int max_chunk) {
  const int64_t full = ((int64_t)kv_max + 63) / 64 * 64;
  if (d.window <= 0) return (int)full;
  const int64_t need = (int64_t)d.window + max_chunk - 1;
  const int64_t ring = (need + 63) / 64 * 64;
  return (int)(ring < full ? ring : full);
}

int32_t check_layer(const g4attn_stack* st, int32_t layer) {
  if (!st) return fail(G4ATTN_ERR_NULL, "stack is NULL");
  if (layer < 0 || layer >= (int32_t)st->L.size())
    return fail(G4ATTN_ERR_RANGE, "layer %d out of range [0, %zu)", layer, st->L.size());
  return G4ATTN_OK;
}

// Decode split policy: splits hold a fixed number of key blocks, sized so
// that a sequence of the longest (hinted) length uses enough splits for the
// grid to give every CU one workgroup; shorter sequences use fewer.  (Two
// workgroups per CU, which the registers allow, measured slower: the four
// waves of one workgroup already keep enough loads in flight, and twice the
// splits double the partial results and lengthen the merge.)
// A split also writes rows x head_dim fp32 partial outputs (and reads them
// back in the merge); splits are made long enough that these stay within
// an eighth of the split's cache bytes (this binds where many query heads
// share one KV head, e.g. 16 rows over the K-only blocks of k_eq_v layers).
// A split also gets at least one block per wave where the context has them.
// (Planning k_eq_v layers for more, shorter splits or fewer, longer ones
// measured slower in both directions.)
void decode_splits(int keys_max, int KB, int pairs, int rows, int planes, bool aligned_start,
                   int* blocks_per_split, int* n_splits) {
  // a range that may start inside a block spans one block more
  const int nb_max = (keys_max + KB - 1) / KB + (aligned_start ? 0 : 1);
  const int target_wgs = 256;
  int ns = ceil_div(target_wgs, pairs);
  if (ns > g4::kMaxDecodeSplits) ns = g4::kMaxDecodeSplits;
  if (ns > nb_max) ns = nb_max;
  if (ns < 1) ns = 1;
  int bps = ceil_div(nb_max, ns);
  // at least one block for each of a workgroup's 4 waves (short contexts over
  // few sequences: fewer, fuller splits and a merge small enough to stay in
  // the kernel)
  if (bps < 4) bps = nb_max < 4 ? nb_max : 4;
  // partial bytes per split: rows * D * 4; cache bytes per block: KB * D * 2 * planes
  const int min_bps = ceil_div(8 * rows * 4, KB * 2 * planes);
  if (ns > 1 && bps < min_bps) bps = min_bps;
  if (bps < ceil_div(nb_max, g4::kMaxDecodeSplits)) bps = ceil_div(nb_max, g4::kMaxDecodeSplits);
  *blocks_per_split = bps;
  *n_splits = ceil_div(nb_max, bps);
}

// Split results are merged by the last workgroup to arrive when the merge is
// small (its partials within kInKernelMergeBytes, at most
// kMaxInKernelSplits splits: that workgroup reads two splits per round
// trip); larger merges go to a separate kernel with one thread per four
// dims of a row, sixteen splits per round trip.
constexpr int64_t kInKernelMergeBytes = 64 * 1024;
constexpr int kMaxInKernelSplits = 8;

}  // namespace

extern "C" {

const char* g4attn_last_error(void) { return g_err.c_str(); }

}  // extern "C"

namespace {

// page == 0: the unpaged layout.  Otherwise `page` slots per page and
// n_pages pages per plane; kv_max is then the block table's positions.
int32_t create_impl(const g4attn_layer_desc* layers, int32_t n_layers, int32_t max_batch,
                    int32_t kv_max, int32_t max_chunk, int32_t page, int32_t n_pages,
                    g4attn_stack** out) {
  if (!layers || !out) return fail(G4ATTN_ERR_NULL, "layers and out must be non-NULL");
  if (n_layers <= 0) return fail(G4ATTN_ERR_DESC, "n_layers must be positive");
  if (max_batch <= 0 || max_batch > 65535) return fail(G4ATTN_ERR_DESC, "max_batch %d", max_batch);
  if (kv_max <= 0 || kv_max > (1 << 24)) return fail(G4ATTN_ERR_DESC, "kv_max %d", kv_max);
  if (max_chunk <= 0 || max_chunk > 4096) return fail(G4ATTN_ERR_DESC, "max_chunk %d", max_chunk);

  g4attn_stack* st = new (std::nothrow) g4attn_stack();
  if (!st) return fail(G4ATTN_ERR_DESC, "out of host memory");
  st->max_batch = max_batch;
  st->kv_max = kv_max;
  st->max_chunk = max_chunk;
  st->paged = page > 0;
  st->page = page;
  st->n_pages = n_pages;
  st->L.resize(n_layers);

  for (int i = 0; i < n_layers; ++i) {
    const g4attn_layer_desc& d = layers[i];
    int32_t rc = G4ATTN_OK;
    if (d.n_q_heads <= 0 || d.n_kv_heads <= 0)
      rc = fail(G4ATTN_ERR_DESC, "layer %d: head counts must be positive", i);
    else if (d.n_q_heads % d.n_kv_heads != 0)
      rc = fail(G4ATTN_ERR_DESC, "layer %d: n_q_heads %d not a multiple of n_kv_heads %d", i,
                d.n_q_heads, d.n_kv_heads);
    else if (d.n_q_heads > 4096)
      rc = fail(G4ATTN_ERR_DESC, "layer %d: too many heads", i);
    else if (d.window < 0)
      rc = fail(G4ATTN_ERR_DESC, "layer %d: window %d < 0", i, d.window);
    else if (d.k_eq_v != 0 && d.k_eq_v != 1)
      rc = fail(G4ATTN_ERR_DESC, "layer %d: k_eq_v must be 0 or 1", i);
    else if (!std::isfinite(d.scale))
      rc = fail(G4ATTN_ERR_DESC, "layer %d: scale is not finite", i);
    else if (!(d.softcap == 0.f ||
               (d.softcap > 0.f && std::isfinite(d.softcap) && std::isfinite(d.scale / d.softcap) &&
                std::isfinite(d.softcap * 1.4426950408889634f))))
      rc = fail(G4ATTN_ERR_DESC, "layer %d: softcap must be 0 or positive and finite, with "
                "scale / softcap finite", i);
    else if (!head_dim_supported(d.head_dim))
      rc = fail(G4ATTN_ERR_UNSUPPORTED, "layer %d: head_dim %d not built (32/64/128/256/512)", i,
                d.head_dim);
    if (rc != G4ATTN_OK) {
      delete st;
      return rc;
    }
    int owner = i;
    if (d.kv_owner_layer != -1 && d.kv_owner_layer != i) {
      const int o = d.kv_owner_layer;
      if (o < 0 || o >= i) {
        delete st;
        return fail(G4ATTN_ERR_OWNER, "layer %d: owner %d is not an earlier layer", i, o);
      }
      const g4attn_layer_desc& od = layers[o];
      if (od.kv_owner_layer != -1 && od.kv_owner_layer != o) {
        delete st;
        return fail(G4ATTN_ERR_OWNER, "layer %d: owner %d is itself KV-shared", i, o);
      }
      if (od.n_kv_heads != d.n_kv_heads || od.head_dim != d.head_dim ||
          od.k_eq_v != d.k_eq_v || od.window != d.window) {
        delete st;
        return fail(G4ATTN_ERR_OWNER,
                    "layer %d: (n_kv_heads, head_dim, k_eq_v, window) differ from owner %d", i,
                    o);
      }
      owner = o;
    }
    st->L[i].d = d;
    st->L[i].owner = owner;
  }

  // cache planes of owning layers
  uint64_t off = 0;
  for (int i = 0; i < n_layers; ++i) {
    LayerPlan& p = st->L[i];
    if (p.owner != i) continue;
    p.cap = st->paged ? page : layer_cap(p.d, kv_max, max_chunk);
    const uint64_t plane = (uint64_t)(st->paged ? n_pages : max_batch) * p.d.n_kv_heads *
                           (uint64_t)p.cap * p.d.head_dim * 2;
    p.k_off = off;
    off = align256(off + plane);
    if (p.d.k_eq_v) {
      p.v_off = p.k_off;
    } else {
      p.v_off = off;
      off = align256(off + plane);
    }
  }
  for (int i = 0; i < n_layers; ++i) {
    LayerPlan& p = st->L[i];
    if (p.owner == i) continue;
    const LayerPlan& o = st->L[p.owner];
    p.cap = o.cap;
    p.k_off = o.k_off;
    p.v_off = o.v_off;
  }
  st->cache_bytes = off;

  // workspace: arrival counters, then (m, l) pairs, then partial outputs
  uint64_t ctr = 0, ml = 0, of = 0;
  for (int i = 0; i < n_layers; ++i) {
    const g4attn_layer_desc& d = st->L[i].d;
    const int G = d.n_q_heads / d.n_kv_heads;
    const uint64_t hblk = (uint64_t)(G + 15) / 16;
    const uint64_t c_d = (uint64_t)max_batch * d.n_kv_heads * hblk;
    const uint64_t r_d = (uint64_t)max_batch * d.n_q_heads * g4::kMaxDecodeSplits;
    ctr = std::max(ctr, c_d);
    ml = std::max(ml, 2 * r_d);
    of = std::max(of, (uint64_t)d.head_dim * r_d);
  }
  st->ctr_count = ctr;
  st->ml_floats = ml;
  st->o_floats = of;
  st->ws_ctr_off = 0;
  st->ws_ml_off = align256(ctr * 4);
  st->ws_o_off = align256(st->ws_ml_off + ml * 4);
  st->ws_bytes = align256(st->ws_o_off + of * 4);

  *out = st;
  return ok();
}

}  // namespace

extern "C" {

int32_t g4attn_stack_create(const g4attn_layer_desc* layers, int32_t n_layers, int32_t max_batch,
                            int32_t kv_max, int32_t max_chunk, g4attn_stack** out) {
  return create_impl(layers, n_layers, max_batch, kv_max, max_chunk, 0, 0, out);
}

int32_t g4attn_stack_create_paged(const g4attn_layer_desc* layers, int32_t n_layers,
                                  int32_t max_batch, int32_t page_size, int32_t n_pages,
                                  int32_t max_pages_per_seq, int32_t max_chunk,
                                  g4attn_stack** out) {
  if (page_size < 64 || page_size % 64 != 0 || page_size > (1 << 16))
    return fail(G4ATTN_ERR_DESC, "page_size %d: a multiple of 64 in [64, 65536]", page_size);
  if (n_pages <= 0) return fail(G4ATTN_ERR_DESC, "n_pages %d must be positive", n_pages);
  if (max_pages_per_seq <= 0 || (int64_t)max_pages_per_seq * page_size > (1 << 24))
    return fail(G4ATTN_ERR_DESC, "max_pages_per_seq %d x page_size %d must be in [1, 2^24]",
                max_pages_per_seq, page_size);
  const int64_t kv_max = (int64_t)max_pages_per_seq * page_size;
  // pages one workgroup's key range may span (its LDS copy of the page ids)
  if (max_chunk > 0 && (kv_max + max_chunk) / page_size + 2 > g4::kMaxWgPages)
    return fail(G4ATTN_ERR_UNSUPPORTED,
                "a key range of %lld positions spans more than %d pages of %d slots",
                (long long)(kv_max + max_chunk), g4::kMaxWgPages - 2, page_size);
  return create_impl(layers, n_layers, max_batch, (int32_t)kv_max, max_chunk, page_size, n_pages,
                     out);
}

void g4attn_stack_destroy(g4attn_stack* stack) { delete stack; }

int32_t g4attn_cache_bytes(const g4attn_stack* st, uint64_t* bytes) {
  if (!st || !bytes) return fail(G4ATTN_ERR_NULL, "stack and bytes must be non-NULL");
  *bytes = st->cache_bytes;
  return ok();
}

int32_t g4attn_workspace_bytes(const g4attn_stack* st, uint64_t* bytes) {
  if (!st || !bytes) return fail(G4ATTN_ERR_NULL, "stack and bytes must be non-NULL");
  *bytes = st->ws_bytes;
  return ok();
}

int32_t g4attn_bind(g4attn_stack* st, void* cache, void* workspace) {
  if (!st || !cache || !workspace)
    return fail(G4ATTN_ERR_NULL, "stack, cache and workspace must be non-NULL");
  if (((uintptr_t)cache & 255) || ((uintptr_t)workspace & 255))
    return fail(G4ATTN_ERR_RANGE, "cache and workspace must be 256-byte aligned");
  st->cache = static_cast<char*>(cache);
  st->ws = static_cast<char*>(workspace);
  return ok();
}

int32_t g4attn_resolve_owner(const g4attn_stack* st, int32_t layer, int32_t* owner) {
  if (int32_t rc = check_layer(st, layer)) return rc;
  if (!owner) return fail(G4ATTN_ERR_NULL, "owner is NULL");
  *owner = st->L[layer].owner;
  return ok();
}

int32_t g4attn_layer_capacity(const g4attn_stack* st, int32_t layer, int32_t* cap) {
  if (int32_t rc = check_layer(st, layer)) return rc;
  if (!cap) return fail(G4ATTN_ERR_NULL, "cap is NULL");
  *cap = st->L[layer].cap;
  return ok();
}

int32_t g4attn_key_range(const g4attn_stack* st, int32_t layer, int64_t q_pos, int64_t n_keys,
                         int64_t* lo, int64_t* hi) {
  if (int32_t rc = check_layer(st, layer)) return rc;
  if (!lo || !hi) return fail(G4ATTN_ERR_NULL, "lo and hi must be non-NULL");
  const int W = st->L[layer].d.window;
  int64_t h = q_pos + 1 < n_keys ? q_pos + 1 : n_keys;
  if (h < 0) h = 0;
  int64_t l = 0;
  if (W > 0) {
    l = q_pos - W + 1;
    if (l < 0) l = 0;
  }
  if (l > h) l = h;
  *lo = l;
  *hi = h;
  return ok();
}

int32_t g4attn_kv_offset(const g4attn_stack* st, int32_t layer, int32_t b, int32_t kv_head,
                         int64_t pos, int32_t d, int64_t* off_k, int64_t* off_v) {
  if (int32_t rc = check_layer(st, layer)) return rc;
  if (!off_k || !off_v) return fail(G4ATTN_ERR_NULL, "off_k and off_v must be non-NULL");
  if (st->paged)
    return fail(G4ATTN_ERR_UNSUPPORTED, "paged stack: positions map through a block table "
                                        "(g4attn_page_offset gives a page's layout)");
  const LayerPlan& p = st->L[layer];
  if (b < 0 || b >= st->max_batch || kv_head < 0 || kv_head >= p.d.n_kv_heads || pos < 0 ||
      pos >= st->kv_max || d < 0 || d >= p.d.head_dim)
    return fail(G4ATTN_ERR_RANGE, "(b %d, kv_head %d, pos %lld, d %d) out of range", b, kv_head,
                (long long)pos, d);
  const int D = p.d.head_dim;
  const int64_t slot = pos % p.cap;
  const int64_t seg = ((int64_t)b * p.d.n_kv_heads + kv_head) * p.cap * D * 2;
  *off_k = (int64_t)p.k_off + seg + g4::k_elem_offset(slot, d, D);
  *off_v = p.d.k_eq_v ? *off_k : (int64_t)p.v_off + seg + g4::v_elem_offset(slot, d, D);
  return ok();
}

int32_t g4attn_page_offset(const g4attn_stack* st, int32_t layer, int32_t page, int32_t kv_head,
                           int32_t slot, int32_t d, int64_t* off_k, int64_t* off_v) {
  if (int32_t rc = check_layer(st, layer)) return rc;
  if (!off_k || !off_v) return fail(G4ATTN_ERR_NULL, "off_k and off_v must be non-NULL");
  if (!st->paged) return fail(G4ATTN_ERR_UNSUPPORTED, "stack is not paged");
  const LayerPlan& p = st->L[layer];
  if (page < 0 || page >= st->n_pages || kv_head < 0 || kv_head >= p.d.n_kv_heads || slot < 0 ||
      slot >= st->page || d < 0 || d >= p.d.head_dim)
    return fail(G4ATTN_ERR_RANGE, "(page %d, kv_head %d, slot %d, d %d) out of range", page,
                kv_head, slot, d);
  const int D = p.d.head_dim;
  const int64_t seg = ((int64_t)page * p.d.n_kv_heads + kv_head) * st->page * D * 2;
  *off_k = (int64_t)p.k_off + seg + g4::k_elem_offset(slot, d, D);
  *off_v = p.d.k_eq_v ? *off_k : (int64_t)p.v_off + seg + g4::v_elem_offset(slot, d, D);
  return ok();
}

}  // extern "C"

namespace {

g4::PageTable page_table(const g4attn_stack* st, const int32_t* table) {
  g4::PageTable t{};
  if (st->paged) {
    t.table = table;
    t.stride = st->kv_max / st->page;
    t.page = st->page;
    t.n_pages = st->n_pages;
  }
  return t;
}

// The current token's rows for a fused decode step: K always, V exactly when
// the layer has a V plane.
int32_t check_new_rows(const LayerPlan& p, const void* k_new, const void* v_new) {
  if (!k_new) return fail(G4ATTN_ERR_NULL, "k_new must be non-NULL");
  if (p.d.k_eq_v && v_new) return fail(G4ATTN_ERR_NULL, "v_new must be NULL on a k_eq_v layer");
  if (!p.d.k_eq_v && !v_new) return fail(G4ATTN_ERR_NULL, "v_new must be non-NULL");
  return G4ATTN_OK;
}

// The paged and unpaged entry points take the same arguments but for the
// block table; each accepts only its own kind of stack.
int32_t check_mode(const g4attn_stack* st, const int32_t* table, bool paged_call) {
  if (paged_call && !st->paged)
    return fail(G4ATTN_ERR_UNSUPPORTED, "stack is not paged: use the unpaged entry point");
  if (!paged_call && st->paged)
    return fail(G4ATTN_ERR_UNSUPPORTED, "stack is paged: use the _paged entry point");
  if (paged_call && !table) return fail(G4ATTN_ERR_NULL, "block_table must be non-NULL");
  return G4ATTN_OK;
}

int32_t append_impl(const g4attn_stack* st, int32_t layer, const void* k, const void* v,
                    const int32_t* start_pos, const int32_t* n_valid, int32_t batch,
                    int32_t n_new, int32_t max_end_pos, const int32_t* table, void* stream) {
  const LayerPlan& p = st->L[layer];
  if (p.owner != layer)
    return fail(G4ATTN_ERR_SHARED_LAYER, "layer %d reads layer %d's cache and writes none", layer,
                p.owner);
  if (!k || !start_pos) return fail(G4ATTN_ERR_NULL, "k and start_pos must be non-NULL");
  if (p.d.k_eq_v && v) return fail(G4ATTN_ERR_NULL, "v must be NULL on a k_eq_v layer");
  if (!p.d.k_eq_v && !v) return fail(G4ATTN_ERR_NULL, "v must be non-NULL");
  if (batch <= 0 || batch > st->max_batch)
    return fail(G4ATTN_ERR_RANGE, "batch %d not in [1, %d]", batch, st->max_batch);
  if (n_new <= 0 || n_new > st->max_chunk)
    return fail(G4ATTN_ERR_RANGE, "n_new %d not in [1, %d]", n_new, st->max_chunk);
  if (max_end_pos < 0 || max_end_pos > st->kv_max)
    return fail(G4ATTN_ERR_RANGE, "max_end_pos %d not in [0, kv_max=%d]", max_end_pos,
                st->kv_max);
  if (!st->cache || !st->ws) return fail(G4ATTN_ERR_UNBOUND, "cache/workspace not bound");
  g4::AppendArgs a;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.kp = reinterpret_cast<uint16_t*>(st->cache + p.k_off);
  a.vp = p.d.k_eq_v ? nullptr : reinterpret_cast<uint16_t*>(st->cache + p.v_off);
  a.start = start_pos;
  a.nvalid = n_valid;
  a.n_new = n_new;
  a.n_kv = p.d.n_kv_heads;
  a.D = p.d.head_dim;
  a.cap = p.cap;
  a.kv_max = st->kv_max;
  a.pt = page_table(st, table);
  hipError_t e = g4::launch_append(a, batch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(G4ATTN_ERR_HIP, "append launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int32_t g4attn_append_kv(const g4attn_stack* st, int32_t layer, const void* k, const void* v,
                         const int32_t* start_pos, const int32_t* n_valid, int32_t batch,
                         int32_t n_new, int32_t max_end_pos, void* stream) {
  if (int32_t rc = check_layer(st, layer)) return rc;
  if (int32_t rc = check_mode(st, nullptr, false)) return rc;
  return append_impl(st, layer, k, v, start_pos, n_valid, batch, n_new, max_end_pos, nullptr,
                     stream);
}

int32_t g4attn_append_kv_paged(const g4attn_stack* st, int32_t layer, const void* k,
                               const void* v, const int32_t* start_pos, const int32_t* n_valid,
                               int32_t batch, int32_t n_new, int32_t max_end_pos,
                               const int32_t* block_table, void* stream) {
  if (int32_t rc = check_layer(st, layer)) return rc;
  if (int32_t rc = check_mode(st, block_table, true)) return rc;
  return append_impl(st, layer, k, v, start_pos, n_valid, batch, n_new, max_end_pos, block_table,
                     stream);
}

}  // extern "C"

namespace {

// Decode, optionally writing the current token's K / V rows first (k_new).
// use_scratch: split partials and counters go to the library's own device
// scratch instead of the bound workspace (nothing is allocated either way).
int32_t decode_impl(const g4attn_stack* st, int32_t layer, const void* q, const void* k_new,
                    const void* v_new, const int32_t* seq_lens, int32_t batch,
                    int32_t max_seq_len, const int32_t* table, void* out, void* stream,
                    bool use_scratch = false) {
  if (!q || !seq_lens || !out) return fail(G4ATTN_ERR_NULL, "q, seq_lens and out must be non-NULL");
  if (batch <= 0 || batch > st->max_batch)
    return fail(G4ATTN_ERR_RANGE, "batch %d not in [1, %d]", batch, st->max_batch);
  if (max_seq_len < 1 || max_seq_len > st->kv_max)
    return fail(G4ATTN_ERR_RANGE, "max_seq_len %d not in [1, kv_max=%d]", max_seq_len,
                st->kv_max);
  if (use_scratch ? !st->cache : (!st->cache || !st->ws))
    return fail(G4ATTN_ERR_UNBOUND, use_scratch ? "cache not bound" : "cache/workspace not bound");
  const LayerPlan& p = st->L[layer];
  const g4attn_layer_desc& d = p.d;
  const int G = d.n_q_heads / d.n_kv_heads;
  const int n_hblk = (G + 15) / 16;
  if ((int64_t)d.n_kv_heads * n_hblk > 65535)
    return fail(G4ATTN_ERR_UNSUPPORTED, "n_kv_heads x head blocks exceeds the launch grid");
  const int nh = G < 16 ? G : 16;
  const int keys_max = d.window > 0 && d.window < max_seq_len ? d.window : max_seq_len;
  g4::DecodeArgs a;
  const int KB = g4::kDecodeBlock;
  // key ranges start at 0 (a block edge) unless a window can move their start
  const bool aligned_start = d.window == 0 || d.window >= max_seq_len;
  decode_splits(keys_max, KB, batch * d.n_kv_heads * n_hblk, nh, d.k_eq_v ? 1 : 2, aligned_start,
                &a.blocks_per_split, &a.n_splits);
  a.merge_in_kernel = a.n_splits <= kMaxInKernelSplits &&
                              (int64_t)a.n_splits * nh * d.head_dim * 4 <= kInKernelMergeBytes
                          ? 1
                          : 0;
  // cache bytes this call may read: the hint's keys of every (sequence, KV head)
  const int64_t call_bytes = (int64_t)batch * d.n_kv_heads * keys_max * d.head_dim * 2 *
                             (d.k_eq_v ? 1 : 2);
  a.stream_loads = call_bytes > g4::kStreamLoadBytes ? 1 : 0;
  a.q = static_cast<const uint16_t*>(q);
  a.kp = reinterpret_cast<uint16_t*>(st->cache + p.k_off);
  a.vp = reinterpret_cast<uint16_t*>(st->cache + p.v_off);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.seq_lens = seq_lens;
  a.out = static_cast<uint16_t*>(out);
  if (use_scratch) {
    // counters first, then (m, l) pairs and partial outputs sized for this
    // call's split plan (a single split writes its output directly and
    // touches neither)
    const uint64_t n_ctr = a.n_splits > 1 ? (uint64_t)batch * d.n_kv_heads * n_hblk : 0;
    const uint64_t rows = a.n_splits > 1 ? (uint64_t)batch * d.n_q_heads * a.n_splits : 0;
    const uint64_t ml_bytes = align256(rows * 2 * 4);
    const uint64_t need = g4::kScratchCounterBytes + ml_bytes + rows * d.head_dim * 4;
    if (n_ctr * 4 > g4::kScratchCounterBytes || need > g4::kScratchBytes)
      return fail(G4ATTN_ERR_UNSUPPORTED,
                  "layer %d: this call needs %llu bytes of decode scratch (%llu counters); the "
                  "library holds %llu bytes (%llu counters) per GPU",
                  layer, (unsigned long long)need, (unsigned long long)n_ctr,
                  (unsigned long long)g4::kScratchBytes,
                  (unsigned long long)(g4::kScratchCounterBytes / 4));
    void* base = nullptr;
    bool first = false;
    hipError_t e = g4::scratch_address(&base, &first);
    if (e != hipSuccess)
      return fail(G4ATTN_ERR_HIP, "decode scratch address: %s", hipGetErrorString(e));
    char* sc = static_cast<char*>(base);
    if (first) {  // the kernels leave the counters at zero after every call
      e = g4::launch_zero(reinterpret_cast<int32_t*>(sc), (int)(g4::kScratchCounterBytes / 4),
                          static_cast<hipStream_t>(stream));
      if (e != hipSuccess)
        return fail(G4ATTN_ERR_HIP, "decode scratch clear: %s", hipGetErrorString(e));
    }
    a.counters = reinterpret_cast<int32_t*>(sc);
    a.part_ml = reinterpret_cast<float*>(sc + g4::kScratchCounterBytes);
    a.part_o = reinterpret_cast<float*>(sc + g4::kScratchCounterBytes + ml_bytes);
  } else {
    a.counters = reinterpret_cast<int32_t*>(st->ws + st->ws_ctr_off);
    a.part_ml = reinterpret_cast<float*>(st->ws + st->ws_ml_off);
    a.part_o = reinterpret_cast<float*>(st->ws + st->ws_o_off);
  }
  a.n_q = d.n_q_heads;
  a.n_kv = d.n_kv_heads;
  a.G = G;
  a.n_hblk = n_hblk;
  a.cap = p.cap;
  a.window = d.window;
  a.kv_max = st->kv_max;
  a.max_len = max_seq_len;
  a.scale_log2 = d.scale * 1.4426950408889634f;
  a.softcap = d.softcap > 0.f ? 1 : 0;
  a.cap_in = a.softcap ? d.scale / d.softcap : 0.f;
  a.cap_log2 = a.softcap ? d.softcap * 1.4426950408889634f : 0.f;
  a.pt = page_table(st, table);
  hipError_t e = g4::launch_decode(d.head_dim, d.k_eq_v != 0, a, batch,
                                   static_cast<hipStream_t>(stream));
  if (e == hipSuccess && a.n_splits > 1 && !a.merge_in_kernel) {
    g4::MergeArgs m{};
    m.part_o = a.part_o;
    m.part_ml = a.part_ml;
    m.out = a.out;
    m.rows = batch * d.n_q_heads;
    m.n_splits = a.n_splits;
    m.D = d.head_dim;
    m.n_q = d.n_q_heads;
    m.seq_lens = seq_lens;
    m.window = d.window;
    m.kv_max = st->kv_max;
    m.max_len = max_seq_len;
    m.KB = KB;
    m.blocks_per_split = a.blocks_per_split;
    e = g4::launch_merge(m, static_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess) return fail(G4ATTN_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int32_t g4attn_decode(const g4attn_stack* st, int32_t layer, const void* q,
                      const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, void* out,
                      void* stream) {
  if (int32_t rc = check_layer(st, layer)) return rc;
  if (int32_t rc = check_mode(st, nullptr, false)) return rc;
  return decode_impl(st, layer, q, nullptr, nullptr, seq_lens, batch, max_seq_len, nullptr, out,
                     stream);
}

int32_t g4attn_decode_noalloc(const g4attn_stack* st, int32_t layer, const void* q,
                              const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                              void* out, void* stream) {
  if (int32_t rc = check_layer(st, layer)) return rc;
  if (int32_t rc = check_mode(st, nullptr, false)) return rc;
  return decode_impl(st, layer, q, nullptr, nullptr, seq_lens, batch, max_seq_len, nullptr, out,
                     stream, true);
}

int32_t g4attn_decode_paged(const g4attn_stack* st, int32_t layer, const void* q,
                            const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                            const int32_t* block_table, void* out, void* stream) {
  if (int32_t rc = check_layer(st, layer)) return rc;
  if (int32_t rc = check_mode(st, block_table, true)) return rc;
  return decode_impl(st, layer, q, nullptr, nullptr, seq_lens, batch, max_seq_len, block_table,
                     out, stream);
}

int32_t g4attn_decode_append(const g4attn_stack* st, int32_t layer, const void* q,
                             const void* k_new, const void* v_new, const int32_t* seq_lens,
                             int32_t batch, int32_t max_seq_len, void* out, void* stream) {
  if (int32_t rc = check_layer(st, layer)) return rc;
  const LayerPlan& p = st->L[layer];
  if (p.owner != layer)
    return fail(G4ATTN_ERR_SHARED_LAYER, "layer %d reads layer %d's cache and writes none", layer,
                p.owner);
  if (int32_t rc = check_new_rows(p, k_new, v_new)) return rc;
  if (int32_t rc = check_mode(st, nullptr, false)) return rc;
  return decode_impl(st, layer, q, k_new, v_new, seq_lens, batch, max_seq_len, nullptr, out,
                     stream);
}

int32_t g4attn_decode_append_paged(const g4attn_stack* st, int32_t layer, const void* q,
                                   const void* k_new, const void* v_new,
                                   const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                   const int32_t* block_table, void* out, void* stream) {
  if (int32_t rc = check_layer(st, layer)) return rc;
  if (int32_t rc = check_mode(st, block_table, true)) return rc;
  const LayerPlan& p = st->L[layer];
  if (p.owner != layer)
    return fail(G4ATTN_ERR_SHARED_LAYER, "layer %d reads layer %d's cache and writes none", layer,
                p.owner);
  if (int32_t rc = check_new_rows(p, k_new, v_new)) return rc;
  return decode_impl(st, layer, q, k_new, v_new, seq_lens, batch, max_seq_len, block_table, out,
                     stream);
}

static int32_t prefill_impl(const g4attn_stack* st, int32_t layer, const void* q,
                            const int32_t* start_pos, int32_t batch, int32_t n_tok,
                            int32_t max_start_pos, const int32_t* table, void* out,
                            void* stream) {
  if (!q || !start_pos || !out)
    return fail(G4ATTN_ERR_NULL, "q, start_pos and out must be non-NULL");
  if (batch <= 0 || batch > st->max_batch)
    return fail(G4ATTN_ERR_RANGE, "batch %d not in [1, %d]", batch, st->max_batch);
  if (n_tok <= 0 || n_tok > st->max_chunk)
    return fail(G4ATTN_ERR_RANGE, "n_tok %d not in [1, %d]", n_tok, st->max_chunk);
  if (max_start_pos < 0 || (int64_t)max_start_pos + n_tok > st->kv_max)
    return fail(G4ATTN_ERR_RANGE, "max_start_pos %d + n_tok %d exceeds kv_max %d", max_start_pos,
                n_tok, st->kv_max);
  if (!st->cache || !st->ws) return fail(G4ATTN_ERR_UNBOUND, "cache/workspace not bound");
  const LayerPlan& p = st->L[layer];
  const g4attn_layer_desc& d = p.d;
  const int G = d.n_q_heads / d.n_kv_heads;
  g4::PrefillArgs a;
  a.rows = n_tok * G;
  a.n_rowblk = (a.rows + g4::kPrefillRows - 1) / g4::kPrefillRows;
  if ((int64_t)batch * d.n_kv_heads * a.n_rowblk + 7 > (int64_t)INT32_MAX)
    return fail(G4ATTN_ERR_UNSUPPORTED, "prefill grid of %lld workgroups too large",
                (long long)batch * d.n_kv_heads * a.n_rowblk);
  a.q = static_cast<const uint16_t*>(q);
  a.kp = reinterpret_cast<const uint16_t*>(st->cache + p.k_off);
  a.vp = reinterpret_cast<const uint16_t*>(st->cache + p.v_off);
  a.start_pos = start_pos;
  a.out = static_cast<uint16_t*>(out);
  a.batch = batch;
  a.n_q = d.n_q_heads;
  a.n_kv = d.n_kv_heads;
  a.G = G;
  a.T = n_tok;
  a.cap = p.cap;
  a.window = d.window;
  a.kv_max = st->kv_max;
  a.max_start = max_start_pos;
  a.scale_log2 = d.scale * 1.4426950408889634f;
  a.softcap = d.softcap > 0.f ? 1 : 0;
  a.cap_in = a.softcap ? d.scale / d.softcap : 0.f;
  a.cap_log2 = a.softcap ? d.softcap * 1.4426950408889634f : 0.f;
  a.pt = page_table(st, table);
  hipError_t e = g4::launch_prefill(d.head_dim, d.k_eq_v != 0, a,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(G4ATTN_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return ok();
}

int32_t g4attn_prefill(const g4attn_stack* st, int32_t layer, const void* q,
                       const int32_t* start_pos, int32_t batch, int32_t n_tok,
                       int32_t max_start_pos, void* out, void* stream) {
  if (int32_t rc = check_layer(st, layer)) return rc;
  if (int32_t rc = check_mode(st, nullptr, false)) return rc;
  return prefill_impl(st, layer, q, start_pos, batch, n_tok, max_start_pos, nullptr, out, stream);
}

int32_t g4attn_prefill_paged(const g4attn_stack* st, int32_t layer, const void* q,
                             const int32_t* start_pos, int32_t batch, int32_t n_tok,
                             int32_t max_start_pos, const int32_t* block_table, void* out,
                             void* stream) {
  if (int32_t rc = check_layer(st, layer)) return rc;
  if (int32_t rc = check_mode(st, block_table, true)) return rc;
  return prefill_impl(st, layer, q, start_pos, batch, n_tok, max_start_pos, block_table, out,
                      stream);
}

}  // extern "C"
