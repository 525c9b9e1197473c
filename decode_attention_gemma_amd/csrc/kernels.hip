// HIP kernels for gfx950 (MI355X): KV append, split-K decode, split merge,
// and a causal / sliding prefill chunk, all on bf16 MFMA with fp32 softmax.
//
// The attention computed is the masked softmax attention of Gemma-4's layers:
// query head h reads KV head h / G ("Porting Gemma-4 (2B / 4B / 12B) to AWS
// Inferentia2", 2.2), sliding layers see the last `window` positions and
// global ones all earlier positions (same page, introduction table), and
// k_eq_v layers use the cached K rows as values ("Gemma-4 12B on AWS
// Inferentia2 -- Tensor-Parallel (TP=2), device prefill", "Why this is its own
// port").
//
// Matrix-core operand layout (v_mfma_f32_16x16x32_bf16, q = lane / 16,
// c = lane % 16): A (16 x 32): lane holds row c, k-slots 8q .. 8q+7;
// B (32 x 16): lane holds column c, the same k-slots; D (16 x 16): lane holds
// rows 4q .. 4q+3 of column c.  v_mfma_f32_16x16x16_bf16 is the same with four
// k-slots 4q .. 4q+3.  Scores are computed transposed, S^T = K Q^T (keys as
// rows, query rows as columns), so each lane's accumulator column is one query
// row and the softmax rescale of O^T = V^T P^T is lane-local.  For the PV
// contraction over a 32-key block, hardware k-slot (q, j) carries key 4q + j
// (j < 4) or 16 + 4q + j - 4 (j >= 4): exactly the keys whose scores lane
// (c, q) holds from the two 16-key score blocks, and the order the V plane is
// stored in (see internal.h).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>
#include <mutex>
#include <type_traits>

#include "internal.h"

namespace g4 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();
// log2 of the largest probability the lazily rescaled online softmax admits
constexpr float kLazyRescale = 8.f;
// k_eq_v prefill: query sub-tiles read from LDS per wave ahead of the score
// MFMA that uses them (one ahead; a second one makes the compiler spill)
constexpr int kQueryReadAhead = 2;

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                    __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four lane groups that
// hold one MFMA output column), with the VALU row swaps: no LDS round trip,
// so it does not wait behind the wave's outstanding LDS operations.  After a
// swap of x with itself, one of the two results holds the lane's own value
// and the other its partner's.
__device__ __forceinline__ float max_over_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// tanh for the attention-logit cap.  Below |x| = 1/16 its Taylor series
// through x^7 (the next term is under 4e-13 relative there), so that a cap far
// above the scores returns them unchanged; elsewhere tanh|x| = (1 - e)/(1 + e)
// with e = exp(-2|x|), which tends to exactly +-1 as e underflows.  Relative
// error about 1e-6 (exp2 and reciprocal hardware approximations).
__device__ __forceinline__ float tanh_cap(float x) {
  const float ax = __builtin_fabsf(x);
  const float x2 = x * x;
  const float p = x * (1.f + x2 * (-1.f / 3.f + x2 * (2.f / 15.f + x2 * (-17.f / 315.f))));
  const float e = fast_exp2(-2.8853900817779268f * ax);  // exp(-2|x|)
  const float t = (1.f - e) * __builtin_amdgcn_rcpf(1.f + e);
  return ax < 0.0625f ? p : __builtin_copysignf(t, x);
}

// Scheduling fence: the values in `acc` count as read and rewritten here, and
// memory operations do not move across it.  Loads placed after it therefore
// stay after the instructions that produced `acc`.
template <int N>
__device__ __forceinline__ void pin_after(f32x4 (&acc)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(acc[i])::"memory");
}

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Cache rows: decode reads each KV byte once per call, so where a call reads
// more than the caches hold its loads carry the non-temporal hint (streamed
// past the caches; on a 134 MB layer this takes the sustained read rate from
// about 5.8 to 6.3 TB/s).  Smaller calls keep the default policy, under which
// a cache that fits stays resident from one step to the next.  Prefill
// rereads every key block from L2 across the row blocks of one (sequence, KV
// head), so its loads keep the default policy.
template <bool NT>
__device__ __forceinline__ u32x4 ldc16(const uint16_t* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }


// Split partial results cross workgroups that may run on different XCDs
// (each with its own L2).  They are written and read with the agent-scope
// coherence bit (sc1: write-through / read-around the XCD's L2), the same
// access the compiler emits for agent-scope atomics, and the writer waits for
// the stores to complete before it signals arrival with an agent-scope atomic.
// This avoids the whole-L2 write-back a release fence performs.
__device__ __forceinline__ void st16_coherent(float* p, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 8 bytes read coherently at agent scope (an atomic load: the compiler tracks
// its completion like any other load)
__device__ __forceinline__ uint64_t ld8_coherent(const float* p) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival of one split: returns true in the workgroup that arrived last.  All
// threads must have waited for their partial-result stores (wait_vmem).
__device__ __forceinline__ bool arrive_last(int32_t* ctr, int n, int* s_flag) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = old == n - 1;
  }
  __syncthreads();
  return *s_flag != 0;
}

// ---------------------------------------------------------------------------
// append: scatter new rows into the operand-ordered planes
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
  const int row = blockIdx.x;
  const int b = blockIdx.y;
  const int t = row / a.n_kv;
  const int g = row - t * a.n_kv;
  const int nv = a.nvalid ? a.nvalid[b] : a.n_new;
  if (t >= nv) return;
  const int pos = a.start[b] + t;
  if (pos < 0 || pos >= a.kv_max) return;
  const int D = a.D;
  const size_t src = ((size_t)(b * a.n_new + t) * a.n_kv + g) * D;
  int slot;
  size_t seg;  // elements
  if (a.pt.table) {
    const int pg = clamp_page(a.pt.table[(size_t)b * a.pt.stride + pos / a.pt.page], a.pt.n_pages);
    slot = pos % a.pt.page;
    seg = ((size_t)pg * a.n_kv + g) * a.pt.page * D;
  } else {
    slot = pos % a.cap;
    seg = (size_t)(b * a.n_kv + g) * a.cap * D;
  }
  // K: each 8-dim chunk is 16 contiguous bytes
  for (int c = threadIdx.x; c < D / 8; c += 64) {
    const int d = 8 * c;
    const int64_t off = k_elem_offset(slot, d, D) / 2;
    *reinterpret_cast<u32x4*>(a.kp + seg + off) = ldg16(a.k + src + d);
  }
  if (a.vp) {
    for (int d = threadIdx.x; d < D; d += 64)
      a.vp[seg + v_elem_offset(slot, d, D) / 2] = a.v[src + d];
  }
}

// ---------------------------------------------------------------------------
// split merge: out[row] = sum_s w_s O_s / sum_s w_s l_s, w_s = 2^(m_s - max m)
// ---------------------------------------------------------------------------


// Stand-alone version for large decode merges (a kernel boundary separates
// writer and reader, so ordinary loads see the partials).  A workgroup takes
// R = max(64, D/4) / (D/4) rows; every thread owns one 4-dim slice of a row.
// A thread reads the (m, l) pairs and its slices of the partial outputs of up
// to CH splits at once, all from its own row's slots, and merges them in
// registers: no LDS, no barrier.  The first CH splits' loads go out together
// with the sequence length (their addresses do not depend on it; slots past
// the row's splits are read and ignored), so a row of at most CH splits
// takes one memory round trip.
template <int D>
__global__ __launch_bounds__(D / 4 > 64 ? D / 4 : 64) void merge_kernel(MergeArgs a) {
  constexpr int D4 = D / 4;
  constexpr int NT = D4 > 64 ? D4 : 64;
  constexpr int R = NT / D4;
  constexpr int CH = 16;  // splits per round trip
  const int tid = threadIdx.x;
  const int r_me = tid / D4;  // R * D4 == NT
  const int d = 4 * (tid - r_me * D4);
  const int row = blockIdx.x * R + r_me;
  if (row >= a.rows) return;
  const float* pml = a.part_ml + (size_t)row * a.n_splits * 2;
  const float* po = a.part_o + (size_t)row * a.n_splits * D + d;
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 ml[CH];
  f32x4 v[CH];
  // splits s0 .. s0 + CH - 1, indices clamped to `last` (repeats hit in cache)
  auto load_batch = [&](int s0, int last) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int si = min(s0 + i, last);
      ml[i] = *reinterpret_cast<const f32x2*>(pml + (size_t)si * 2);
      v[i] = *reinterpret_cast<const f32x4*>(po + (size_t)si * D);
    }
  };
  load_batch(0, a.n_splits - 1);
  int L = a.seq_lens[row / a.n_q];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  const int lo = a.window > 0 ? max(0, L - a.window) : 0;
  int n, f, e;
  decode_split_range(lo, L, a.KB, a.blocks_per_split, 0, &n, &f, &e);
  if (n <= 1) return;  // written by the decode kernel itself
  n = min(n, a.n_splits);
  float M = kNegInf, lsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n; s0 += CH) {
    if (s0 > 0) load_batch(s0, n - 1);
    // out = sum_s w_s O_s / sum_s w_s l_s, w_s = 2^(m_s - max m) over the
    // splits with keys, in split order; rescaled when a batch raises the max
    float bm = M;
#pragma unroll
    for (int i = 0; i < CH; ++i)
      if (s0 + i < n && ml[i][1] > 0.f) bm = fmaxf(bm, ml[i][0]);
    if (bm != M) {
      const float sc = fast_exp2(M - bm);  // 0 while nothing was added
      acc *= sc;
      lsum *= sc;
      M = bm;
    }
#pragma unroll
    for (int i = 0; i < CH; ++i)
      if (s0 + i < n && ml[i][1] > 0.f) {
        const float w = fast_exp2(ml[i][0] - M);
        lsum += w * ml[i][1];
        acc += w * v[i];
      }
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  bf16x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = (__bf16)(acc[j] * inv);
  *reinterpret_cast<bf16x4*>(a.out + (size_t)row * D + d) = o;
}

// ---------------------------------------------------------------------------
// attention over cached key blocks: decode and prefill share one kernel body
// ---------------------------------------------------------------------------
//
// A workgroup owns up to 16 query rows and a range of key blocks (KB keys:
// 32, or 16 on k_eq_v layers).  Wave w of NW takes blocks w, w+NW, ...: it
// streams each block straight from the cache into registers in operand order
// (1 KiB contiguous per load instruction), computes S^T = K Q^T on MFMA with
// the queries read from LDS, keeps its own online-softmax state per row, and
// accumulates O^T = V^T P^T.  On k_eq_v layers the K block is the V block as
// well: it is staged in a wave-private LDS area and read back transposed with
// ds_read_b64_tr_b16.  No barrier is needed until the NW waves combine their
// states through LDS at the end; latency is hidden by occupancy.
//
// Decode (one query position per sequence): the rows are the query heads of
// one KV head; the sequence's blocks are split over workgroups in proportion
// to its length and the splits are merged (in-kernel or by merge_kernel).
// Prefill (a chunk of T tokens): the rows are 16 consecutive (token, head)
// pairs of one KV head, each with its own causal / sliding window; one
// workgroup streams the whole key range its rows can see, so no split
// results exist.  The grid is laid out so that the row blocks of one
// (sequence, KV head) run on the same XCD and share its L2.

template <int D, bool KEQV, int NW, bool SAG, bool PREFILL>
struct Shape {
  // keys per block: 32, or 16 for k_eq_v prefill, whose staging area holds
  // a whole block per wave
  static constexpr int KB = SAG ? 16 : 32;
  static constexpr int NSB = KB / 16;        // 16-key score blocks per block
  static constexpr int KS = D / 32;          // 1 KiB K sub-tiles per 16 keys
  static constexpr int NDB = D / 16;         // 16-dim output blocks
  // k_eq_v: the block is transposed through LDS in NPH phases of TRH
  // sub-tiles, or staged whole while the scores are computed (SAG)
  static constexpr int TRH = SAG || KS < 2 ? KS : KS / 2;
  static constexpr int NPH = KS / TRH;
  static constexpr int TR_ELEMS = KEQV ? NSB * TRH * 512 : 0;  // per-wave transpose area
  // cross-wave reduction rows are padded by 4 floats so that the 16 rows a
  // wave writes at once start on different LDS banks
  static constexpr int RED_STRIDE = D + 4;
  static constexpr int SLOT_BYTES = 16 * RED_STRIDE * 4;
  static constexpr int TR_BYTES = NW * TR_ELEMS * 2;
  static constexpr int Q_BYTES = KS * 512 * 2;
  // The waves combine their partial outputs in NSL reduction slots: one per
  // wave (one barrier), one per pair of waves (two), or a single slot that
  // the waves add into one after another.  Slots share the LDS with the
  // transpose area.  Both grids are planned for one workgroup per CU, which
  // may then use most of the LDS (the head_dim 512 decode combine takes one
  // barrier instead of four; smaller shapes stay small enough for two).
  static constexpr int BUDGET = 150 * 1024;
  static constexpr int cmax(int a, int b) { return a > b ? a : b; }
  static constexpr bool fits(int n) {
    return cmax(TR_BYTES, n * SLOT_BYTES) + Q_BYTES + 1024 <= BUDGET;
  }
  static constexpr int NSL = fits(NW) ? NW : (NW % 2 == 0 && fits(NW / 2)) ? NW / 2 : 1;
  static constexpr int LDS_BYTES = cmax(TR_BYTES, NSL * SLOT_BYTES);
};

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// FUSED: the decode step that first writes the current token's K/V rows into
// the cache (g4attn_decode_append); its own instances, so that the plain
// decode carries none of that code.
template <int D, bool KEQV, int NW, bool PREFILL, bool PAGED, bool CAP, bool NTL, bool FUSED>
__global__ __launch_bounds__(NW * 64, waves_per_simd(D, KEQV, PREFILL)) void attend_kernel(
    DecodeArgs da, PrefillArgs pa) {
  static_assert(!(FUSED && PREFILL), "the token append is a decode step");
  // k_eq_v prefill stages each K sub-tile for the V^T transpose as soon as
  // its score MFMA has read it, and reloads the register with the next
  // block's sub-tile at once (a whole block of prefetch distance; the staging
  // area then holds a full block per wave)
  constexpr bool SAG = PREFILL && KEQV;
  using S = Shape<D, KEQV, NW, SAG, PREFILL>;
  constexpr int KB = S::KB, NSB = S::NSB, KS = S::KS, NDB = S::NDB;
  constexpr int D4 = D / 4;
  constexpr int NT = NW * 64;

  __shared__ __attribute__((aligned(16))) unsigned char lds[S::LDS_BYTES];
  __shared__ __attribute__((aligned(16))) uint16_t Qs[KS * 512];
  __shared__ float wm[NW][16], wl[NW][16], hM[16], hL[16];
  __shared__ int s_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int c16 = lane & 15;
  const int q4 = lane >> 4;

  // ---- work of this workgroup -------------------------------------------
  int b, g, cap, n_kv;
  int blk_first, blk_end;   // key blocks it streams
  int r_beg, r_end;         // keys it may read; values outside are zeroed
  int full_lo, full_hi;     // keys visible to every valid row
  int row_lo, row_hi;       // keys visible to this lane's row (column c16)
  int nrows;                // valid rows (heads / token-head pairs)
  bool row_ok;
  const uint16_t* qrow;     // this lane's query row
  float scale_log2;
  float cap_in = 0.f, cap_log2 = 0.f;  // attention-logit cap (CAP)
  // decode only
  int split = 0, n_used = 1, head0 = 0, hblk = 0;
  int new_pos = -1;  // fused append: position of the current token in this split
  // prefill only
  int row0 = 0, t_row = 0, h_row = 0;
  int rot = 0;  // this row block's offset into its block range
  int pg_row = 0;  // paged decode: block-table entry `tid` of the sequence
  // This wave's share of the query operand (sub-tiles w, w + NW, ...),
  // loaded before anything that depends on the sequence lengths or
  // positions: it is then in flight during the length read instead of queued
  // behind the first key block (loads complete in issue order).
  constexpr int QPW = (KS + NW - 1) / NW;
  u32x4 qv[QPW];
  auto load_q = [&]() {
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      const int s = w + i * NW;
      // Decode: unconditional, since after a conditional load the compiler
      // cannot count the loads in flight, and its later waits would cover
      // the queries too.  Lanes past the last row read a valid row; each row
      // is its own column of the MFMAs and only valid rows are written out.
      // (Prefill keeps zeros there: the unconditional form spills.)
      if (QPW * NW == KS || s < KS)
        qv[i] = PREFILL && !row_ok ? u32x4{0u, 0u, 0u, 0u} : ldg16(qrow + 32 * s + 8 * q4);
    }
  };
  if constexpr (!PREFILL) {
    const DecodeArgs& a = da;
    split = blockIdx.x;
    g = blockIdx.y / a.n_hblk;
    hblk = blockIdx.y - g * a.n_hblk;
    b = blockIdx.z;
    cap = a.cap;
    n_kv = a.n_kv;
    scale_log2 = a.scale_log2;
    cap_in = a.cap_in;
    cap_log2 = a.cap_log2;
    head0 = g * a.G + hblk * 16;
    nrows = min(16, a.G - hblk * 16);
    row_ok = c16 < nrows;
    qrow = a.q + ((size_t)b * a.n_q + head0 + (row_ok ? c16 : 0)) * D;
    if constexpr (PAGED) {
      // a block-table row of at most one entry per thread is loaded whole,
      // before the queries: its address does not depend on the length, and
      // the waits for it then leave the queries in flight (loads complete in
      // issue order).
      pg_row = a.pt.table[(size_t)b * a.pt.stride + min(tid, a.pt.stride - 1)];
    }
    load_q();
    int L = a.seq_lens[b];
    L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
    const int lo = a.window > 0 ? max(0, L - a.window) : 0;
    decode_split_range(lo, L, KB, a.blocks_per_split, split, &n_used, &blk_first, &blk_end);
    if (split > 0 && split >= n_used) return;  // nothing for this workgroup
    r_beg = max(lo, blk_first * KB);
    r_end = min(L, blk_end * KB);
    full_lo = r_beg;
    full_hi = r_end;
    row_lo = r_beg;
    row_hi = r_end;
    if (FUSED && L > 0 && r_end == L) new_pos = L - 1;
  } else {
    const PrefillArgs& a = pa;
    // physical workgroup p runs on XCD p % 8; give each XCD a contiguous
    // range of logical (sequence, KV head, row block) work
    const int n_log = a.n_rowblk * a.n_kv * a.batch;
    const int per_xcd = (n_log + 7) / 8;  // grid.x == 8 * per_xcd
    const int logical = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (logical >= n_log) return;
    const int rowblk = logical % a.n_rowblk;
    const int grp = logical / a.n_rowblk;
    g = grp % a.n_kv;
    b = grp / a.n_kv;
    cap = a.cap;
    n_kv = a.n_kv;
    scale_log2 = a.scale_log2;
    cap_in = a.cap_in;
    cap_log2 = a.cap_log2;
    row0 = rowblk * 16;
    nrows = min(16, a.rows - row0);
    const int row = row0 + c16;
    row_ok = c16 < nrows;
    t_row = row_ok ? row / a.G : 0;
    h_row = row_ok ? row - t_row * a.G : 0;
    qrow = a.q + (((size_t)b * a.T + t_row) * a.n_q + g * a.G + h_row) * D;
    load_q();
    int start = a.start_pos[b];
    start = start < 0 ? 0 : (start > a.max_start ? a.max_start : start);
    const int p_first = start + row0 / a.G;
    const int p_last = start + (row0 + nrows - 1) / a.G;
    const int p_row = start + t_row;
    auto lo_of = [&](int p) { return a.window > 0 ? max(0, p - a.window + 1) : 0; };
    r_beg = lo_of(p_first);
    r_end = min(p_last + 1, a.kv_max);
    blk_first = r_beg / KB;
    blk_end = r_end > r_beg ? (r_end + KB - 1) / KB : blk_first;
    // The row blocks of one (sequence, KV head) read the same keys.  Each
    // starts at a different place in the range, so that their first rounds
    // together request every block once from HBM and later rounds hit in L2,
    // instead of all of them waiting for the same first touch each round.
    rot = (int)(((long long)rowblk * (blk_end - blk_first)) / a.n_rowblk);
    full_lo = lo_of(p_last);
    full_hi = min(p_first + 1, r_end);
    row_lo = row_ok ? max(lo_of(p_row), r_beg) : 0;
    row_hi = row_ok ? min(p_row + 1, r_end) : 0;
  }
  const int n_keys = r_end - r_beg;
  const uint16_t* kp = PREFILL ? pa.kp : da.kp;
  const uint16_t* vp = PREFILL ? pa.vp : da.vp;
  const size_t seg = (size_t)(b * n_kv + g) * cap * D;  // unpaged segment

  // Paged cache: the page ids of the workgroup's key range, read once into
  // LDS (the range spans at most kMaxWgPages pages; the host checks).
  __shared__ int pg_ids[PAGED ? kMaxWgPages : 1];
  int pg_first = 0;
  if constexpr (PAGED) {
    const PageTable& pt = PREFILL ? pa.pt : da.pt;
    pg_first = (blk_first * KB) / pt.page;
    const int pg_last = blk_end > blk_first ? (blk_end * KB - 1) / pt.page : pg_first;
    const int n_pg = min(pg_last - pg_first + 1, kMaxWgPages);
    const int32_t* row = pt.table + (size_t)b * pt.stride;
    // The row's load (issued whatever the row's size) is waited for here, on
    // every path: otherwise the compiler, which merges what it knows of both
    // paths, waits for it again after the barrier below, together with
    // every load issued after it.
    if constexpr (!PREFILL) asm volatile("" ::"v"(pg_row));
    if (!PREFILL && pt.stride <= NT) {  // the row loaded with the queries
      const int i = tid - pg_first;
      if (tid < pt.stride && i >= 0 && i < n_pg) pg_ids[i] = clamp_page(pg_row, pt.n_pages);
    } else {
      for (int i = tid; i < n_pg; i += NW * 64)
        pg_ids[i] = clamp_page(row[min(pg_first + i, pt.stride - 1)], pt.n_pages);
    }
    __syncthreads();
  }
  // element offset of the segment holding key block blk, and the block's
  // first slot in it
  auto seg_of = [&](int blk, int& slot0) -> size_t {
    if constexpr (!PAGED) {
      slot0 = (blk * KB) % cap;
      return seg;
    } else {
      const int page = PREFILL ? pa.pt.page : da.pt.page;
      const int pos0 = blk * KB;
      slot0 = pos0 % page;
      const int i = min(max(pos0 / page - pg_first, 0), kMaxWgPages - 1);
      return ((size_t)pg_ids[i] * n_kv + g) * page * D;
    }
  };

  // ---- block loads.  The next block's K (and V) is loaded as soon as the
  // registers it lands in are free, so it overlaps the rest of the current
  // block.  With a V plane the wave's last block is peeled off the loop:
  // inside the loop the prefetch is then unconditional, which lets the
  // compiler wait for exactly the loads an instruction needs (memory counters
  // complete in issue order; after a conditional prefetch of the next K, the
  // wait for the current V would also cover the first of those loads) ----
  u32x4 kreg[NSB][KS];
  u32x4 vreg[KEQV ? 1 : NDB];
  // this lane's address in the K sub-tile 0 of a block (sub-tile s of score
  // block sb follows at (sb * KS + s) * 512 elements)
  auto kblock = [&](int blk) {
    int slot0;
    const size_t sg = seg_of(blk, slot0);
    return kp + sg + (size_t)(slot0 / 16) * KS * 512 + lane * 8;
  };
  auto load_k = [&](int blk) {
    const uint16_t* kb = kblock(blk);
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int s = 0; s < KS; ++s) kreg[sb][s] = ldc16<NTL>(kb + (sb * KS + s) * 512);
  };
  auto load_v = [&](int blk) {
    if constexpr (!KEQV) {
      int slot0;
      const uint16_t* vs = vp + seg_of(blk, slot0);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        vreg[db] = ldc16<NTL>(vs + ((size_t)(slot0 / 32) * NDB + db) * 512 + lane * 8);
    }
  };
  const int n_mine = n_keys > 0 && blk_first + w < blk_end
                         ? (blk_end - (blk_first + w) + NW - 1) / NW : 0;  // blocks of this wave
  // fused append: this wave wrote the token's rows and must see its stores
  // complete before the workgroup barrier below
  bool wrote_row = false;
  if constexpr (FUSED) {
    // Fused append: the current token's K (and V) row is written into its
    // cache slot before the wave that reads the token's block (the last block
    // of the range) loads it.  When that block is the reading wave's first,
    // whose loads are issued before the workgroup barrier below, the reader
    // writes the row and waits for its stores before loading anything.
    // Otherwise the next wave writes it and waits for its stores just before
    // the barrier, while its own first block is in flight; the reader loads
    // the token's block after the barrier, late in its stream.  (When the
    // reader wrote and waited every time, the reader, which also streams the
    // most blocks, started its stream a store round trip late.)  No other
    // workgroup of this launch reads that slot as a visible key; several head
    // blocks of one KV head write the same bytes.  The slot's segment is the
    // unpaged one or the page the block table maps the position to.
    const int tok_j = new_pos / KB - blk_first;  // the token block's place in the range
    const int writer = tok_j < NW ? tok_j : (tok_j + 1) % NW;
    if (new_pos >= 0 && w == writer) {
      int slot0;
      const size_t sg = seg_of(new_pos / KB, slot0);
      const int slot = slot0 + new_pos % KB;
      const size_t row = ((size_t)b * n_kv + g) * D;
      // Both rows are loaded before either is stored: one memory round trip.
      // (Loaded and stored element by element, each load stayed behind the
      // store before it, since the two may alias: four round trips.)  Lane l
      // stores the V elements of dims l, l + 64, ...: the 8 lanes that share
      // a 128-byte line of the V plane store in one instruction.
      constexpr int NV = (D + 63) / 64;
      const bool has_k = lane < D / 8;
      u32x4 kc = {0u, 0u, 0u, 0u};
      uint16_t vv[NV];
      if (has_k) kc = ldg16(da.k_new + row + 8 * lane);
      if constexpr (!KEQV) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
          if (lane + 64 * i < D) vv[i] = da.v_new[row + lane + 64 * i];
      }
      if (has_k) *reinterpret_cast<u32x4*>(da.kp + sg + k_elem_offset(slot, 8 * lane, D) / 2) = kc;
      if constexpr (!KEQV) {
        uint16_t* vdst = da.vp + sg;
#pragma unroll
        for (int i = 0; i < NV; ++i)
          if (lane + 64 * i < D) vdst[v_elem_offset(slot, lane + 64 * i, D) / 2] = vv[i];
      }
      if (tok_j < NW)
        wait_vmem();
      else
        wrote_row = true;
    }
  }
  // block of the wave's j-th position in the range (j = w, w + NW, ...)
  const int nblk = blk_end - blk_first;
  auto phys = [&](int j) {
    if constexpr (!PREFILL) {
      return blk_first + j;
    } else {
      int x = j + rot;
      x -= x >= nblk ? nblk : 0;
      return blk_first + x;
    }
  };
  // The first block's loads are issued on every path (a wave without blocks
  // loads one of the range and ignores it): after a conditional load the
  // compiler's wait for the queries would have to cover every load.
  load_k(phys(n_mine > 0 ? w : 0));
  load_v(phys(n_mine > 0 ? w : 0));
  if (wrote_row) {
    // everything older than the first block's loads, the token's row stores
    // included, has landed (vector memory operations complete in issue order)
    constexpr int n_first = NSB * KS + (KEQV ? 0 : NDB);
    constexpr int vm = n_first < 63 ? n_first : 63;
    __builtin_amdgcn_s_waitcnt((vm & 15) | ((vm >> 4) << 14) | 0x0F70);
  }

  // queries as the B operand of S^T = K Q^T (column c16 = row, k-slots =
  // dims), kept in LDS in operand order: sub-tile s, lane L at (s*64 + L)*8
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int s = w + i * NW;
    if (QPW * NW == KS || s < KS) *reinterpret_cast<u32x4*>(&Qs[(s * 64 + lane) * 8]) = qv[i];
  }
  __syncthreads();

  f32x4 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;
  float l_run = 0.f;
  uint16_t* tr = reinterpret_cast<uint16_t*>(lds) + w * S::TR_ELEMS;  // k_eq_v only

  // one key block; `pf` (a bool, or std::true_type / std::false_type) says
  // whether the wave's next block `nxt` is loaded
  auto block = [&](const int blk, const int nxt, auto pf) {
    const bool PFX = pf;  // a compile-time constant where the caller passes a type
    // the next block's address, computed before any compiler barrier below
    // (those make captured values be reloaded)
    const uint16_t* const kbn = kblock(nxt);
    const int pos0 = blk * KB;
    const bool full = pos0 >= full_lo && pos0 + KB <= full_hi;
    const bool vfull = pos0 >= r_beg && pos0 + KB <= r_end;

    // scores, mask, online softmax (lane's column c16 = row).  The compiler
    // barrier keeps the query reads from LDS here instead of hoisting the
    // whole query operand into registers for the loop.  Two independent
    // accumulation chains per score block keep the matrix core busy while
    // each MFMA's result is still in flight.
    asm volatile("" ::: "memory");
    constexpr int NCH = KS >= 2 ? 2 : 1;
    f32x4 sacc[NSB];
    {
      f32x4 sch[NSB][NCH];
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int c = 0; c < NCH; ++c) sch[sb][c] = f32x4{0.f, 0.f, 0.f, 0.f};
      // k_eq_v prefill: query sub-tiles read QD - 1 ahead of their MFMA, so
      // that more than one LDS read is in flight (the staging writes and
      // compiler barriers below would otherwise leave one)
      constexpr int QD = SAG ? kQueryReadAhead : 1;
      bf16x8 qf[QD];
#pragma unroll
      for (int i = 0; i + 1 < QD; ++i)
        qf[i] = *reinterpret_cast<const bf16x8*>(&Qs[(i * 64 + lane) * 8]);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s + QD - 1 < KS)
          qf[(s + QD - 1) % QD] =
              *reinterpret_cast<const bf16x8*>(&Qs[((s + QD - 1) * 64 + lane) * 8]);
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
          sch[sb][s % NCH] = mfma32(as_bf16x8(kreg[sb][s]), qf[s % QD], sch[sb][s % NCH]);
        if constexpr (SAG) {
          // Unconditional: without a next block `nxt` is this block again,
          // an L2 hit.  Behind a run-time condition the compiler no longer
          // counts these loads and, at the fifth sub-tile, waited for the
          // next block's first loads as well: a memory round trip per block.
          *reinterpret_cast<u32x4*>(tr + s * 512 + lane * 8) = kreg[0][s];
          asm volatile("" ::: "memory");  // after the staging write
          kreg[0][s] = ldc16<NTL>(kbn + s * 512);
        }
      }
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        sacc[sb] = sch[sb][0];
#pragma unroll
        for (int c = 1; c < NCH; ++c) sacc[sb] += sch[sb][c];
      }
    }
    if (!KEQV && PFX) {
      // the next K lands in the registers the score MFMAs just read: keep
      // its loads after them (hoisting them would need a second set)
      pin_after(sacc);
      load_k(nxt);
    }
    // visible keys of this lane's row within the block (bitwise, no branches)
    const int vis_lo = full ? INT_MIN : row_lo;
    const int vis_hi = full ? INT_MAX : row_hi;
    float lmax = kNegInf;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kpos = pos0 + 16 * sb + 4 * q4 + j;
        const bool ok = row_ok & (kpos >= vis_lo) & (kpos < vis_hi);
        float sv;
        if constexpr (CAP)  // s * log2(e) with s = c tanh(scale q.k / c)
          sv = cap_log2 * tanh_cap(sacc[sb][j] * cap_in);
        else
          sv = sacc[sb][j] * scale_log2;
        sacc[sb][j] = ok ? sv : kNegInf;
        lmax = fmaxf(lmax, sacc[sb][j]);
      }
    }
    if constexpr (PREFILL) {
      // (decode keeps the shuffles: the row swaps measured no faster there)
      lmax = max_over_lane_groups(lmax);
    } else {
      lmax = fmaxf(lmax, __shfl_xor(lmax, 16));
      lmax = fmaxf(lmax, __shfl_xor(lmax, 32));
    }
    // Lazy rescaling: the reference max m_run moves only when some row's
    // block max exceeds it by more than 2^8, so probabilities stay <= 256
    // (exact enough in fp32 and bf16) and most blocks skip rescaling the
    // output accumulators.  The decision is uniform across the wave.
    // (Only the multiplies sit under the branch: with more inside it the
    // register allocation no longer fits.)
    const bool need = __ballot(lmax > m_run + kLazyRescale) != 0ull;
    const float m_new = need ? fmaxf(m_run, lmax) : m_run;
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
    if (need) {
#pragma unroll
      for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;
    }
    bf16x4 pb[NSB];
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const __bf16 p = (__bf16)fast_exp2(sacc[sb][j] - m_use);
        pb[sb][j] = p;
        psum += (float)p;
      }
    l_run += psum;

    // Values of keys outside [r_beg, r_end) must not reach the MFMA (their
    // probabilities are zero, but the slots may hold any bit pattern).  The
    // mask is per lane and k-slot; it is applied with bitwise ands.
    if constexpr (!KEQV) {
      // P^T as the B operand: k-slot j <-> key 4q+j (j<4) / 16+4q+j-4
      bf16x8 pf8;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pf8[j] = pb[0][j];
        pf8[4 + j] = pb[1][j];
      }
      if (!vfull) {
        u32x4 keep;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          uint32_t m = 0u;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int j = 2 * jj + h;
            const int kpos = pos0 + ((j < 4) ? 4 * q4 + j : 16 + 4 * q4 + j - 4);
            if (kpos >= r_beg && kpos < r_end) m |= 0xffffu << (16 * h);
          }
          keep[jj] = m;
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) vreg[db] &= keep;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(as_bf16x8(vreg[db]), pf8, oacc[db]);
      if (PFX) {
        pin_after(oacc);
        load_v(nxt);
      }
    } else {
      // The K block doubles as V: each phase stages TRH of the sub-tiles of
      // every 16-key half in this wave's LDS area in operand order, after
      // which their registers take the next block's sub-tiles.  One
      // transposing 64-bit read per lane and half then yields
      // V[4q .. 4q+3][d0 + c] of that half for a 16-dim block (the lane
      // addresses key 4q + c/4, dims d0 + 4(c%4) .. +3).  With two halves
      // the two reads form the A operand of a 16x16x32 MFMA whose k-slots
      // carry keys 4q+j / 16+4q+j-4, the order of P^T above.  LDS operations
      // of one wave complete in order.  In a block that reaches outside
      // [r_beg, r_end), the staged rows of those keys are overwritten with
      // zeros (lane L of a sub-tile holds key L % 16 of its half).
      bool key_out[NSB];
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const int kpos = pos0 + 16 * sb + c16;
        key_out[sb] = kpos < r_beg || kpos >= r_end;
      }
      bf16x8 pf8;
      if constexpr (NSB == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pf8[j] = pb[0][j];
          pf8[4 + j] = pb[1][j];
        }
      }
#pragma unroll
      for (int ph = 0; ph < S::NPH; ++ph) {
        if constexpr (!SAG) {
#pragma unroll
          for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int s = 0; s < S::TRH; ++s)
              *reinterpret_cast<u32x4*>(tr + (sb * S::TRH + s) * 512 + lane * 8) =
                  kreg[sb][ph * S::TRH + s];
        }
        if (!SAG && PFX) {
          asm volatile("" ::: "memory");  // after the staging writes
#pragma unroll
          for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int s = 0; s < S::TRH; ++s)
              kreg[sb][ph * S::TRH + s] = ldc16<NTL>(kbn + (sb * KS + ph * S::TRH + s) * 512);
        }
        if (!vfull) {
#pragma unroll
          for (int sb = 0; sb < NSB; ++sb)
            if (key_out[sb]) {
#pragma unroll
              for (int s = 0; s < S::TRH; ++s)
                *reinterpret_cast<u32x4*>(tr + (sb * S::TRH + s) * 512 + lane * 8) =
                    u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int dbl = 0; dbl < NDB / S::NPH; ++dbl) {
          const int dd = 16 * dbl + 4 * (c16 & 3);  // dim within the staged sub-tiles
          const int kk = 4 * q4 + (c16 >> 2);
          uint16_t* src = tr + (dd / 32) * 512 + ((dd % 32) / 8) * 128 + kk * 8 + (dd % 8);
          const int db = ph * (NDB / S::NPH) + dbl;
          const s16x4 raw0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)src);
          if constexpr (NSB == 1) {
            oacc[db] = mfma16(__builtin_bit_cast(bf16x4, raw0), pb[0], oacc[db]);
          } else {
            const s16x4 raw1 =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src + S::TRH * 512));
            // composed as whole 32-bit words (element-wise bf16 inserts
            // were miscompiled into duplicated registers)
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 w0 = __builtin_bit_cast(u32x2, raw0);
            const u32x2 w1 = __builtin_bit_cast(u32x2, raw1);
            const u32x4 va = {w0[0], w0[1], w1[0], w1[1]};
            oacc[db] = mfma32(as_bf16x8(va), pf8, oacc[db]);
          }
        }
      }
    }
  };

  if (n_mine > 0) {
    int j = w;
    if constexpr (KEQV || D >= 512) {
      // k_eq_v decode: no older load is waited for after the next block's
      // loads are issued, so a run-time condition costs nothing (k_eq_v
      // prefill issues them unconditionally).  head_dim 512 with a V plane:
      // a second copy of the body does not fit the registers.
      for (int i = 1; i <= n_mine; ++i, j += NW) block(phys(j), phys(i < n_mine ? j + NW : j), i < n_mine);
    } else {
      for (int i = 1; i < n_mine; ++i, j += NW) block(phys(j), phys(j + NW), std::true_type{});
      block(phys(j), phys(j), std::false_type{});
    }
  }

  // ---- combine the NW waves: common max, rescale, sum through LDS ----
  float lt = l_run;
  lt += __shfl_xor(lt, 16);
  lt += __shfl_xor(lt, 32);
  if (lane < 16) {
    wm[w][lane] = m_run;
    wl[w][lane] = lt;
  }
  __syncthreads();  // also: every wave is done with its transpose area
  float M = kNegInf;
#pragma unroll
  for (int i = 0; i < NW; ++i) M = fmaxf(M, wm[i][c16]);
  const float M_use = M == kNegInf ? 0.f : M;
  if (tid < 16) {
    float Lh = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) Lh += wl[i][tid] * fast_exp2(wm[i][tid] - M_use);
    hM[tid] = M;
    hL[tid] = Lh;
  }
  const float mine = fast_exp2(m_run - M_use);
  constexpr int RS = S::RED_STRIDE;
  constexpr int NSL = S::NSL;
  constexpr int SLOT = 16 * RS;                // floats per slot
  float* red = reinterpret_cast<float*>(lds);  // [NSL][16][RS]
  auto put = [&](int slot, bool add) {         // this wave's rescaled O into a slot
    if (c16 < nrows) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        float* p = red + slot * SLOT + c16 * RS + 16 * db + 4 * q4;
        f32x4 v = oacc[db] * mine;
        if (add) v += *reinterpret_cast<f32x4*>(p);
        *reinterpret_cast<f32x4*>(p) = v;
      }
    }
  };
  if constexpr (NSL == NW) {
    put(w, false);
    __syncthreads();
  } else if constexpr (2 * NSL == NW) {
    if (w >= NSL) put(w - NSL, false);
    __syncthreads();
    if (w < NSL) put(w, true);
    __syncthreads();
  } else {
    for (int step = NW - 1; step >= 0; --step) {
      if (w == step) put(0, step != NW - 1);
      __syncthreads();
    }
  }
  // unnormalised O of this key range: row r, dims d .. d+3
  auto red_sum = [&](int r, int d) {
    f32x4 v = *reinterpret_cast<const f32x4*>(red + r * RS + d);
#pragma unroll
    for (int s = 1; s < NSL; ++s) v += *reinterpret_cast<const f32x4*>(red + s * SLOT + r * RS + d);
    return v;
  };

  // red_sum(r, .) = unnormalised O of this key range for row r; hM, hL per row
  if (PREFILL || n_used <= 1) {
    for (int idx = tid; idx < nrows * D4; idx += NT) {
      const int r = idx / D4;
      const int d = 4 * (idx - r * D4);
      const float il = hL[r] > 0.f ? 1.f / hL[r] : 0.f;
      const f32x4 v = red_sum(r, d);
      bf16x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = (__bf16)(v[j] * il);
      size_t off;
      if constexpr (PREFILL) {
        const int rr = row0 + r;
        const int tt = rr / pa.G;
        off = (((size_t)b * pa.T + tt) * pa.n_q + g * pa.G + (rr - tt * pa.G)) * D;
      } else {
        off = ((size_t)b * da.n_q + head0 + r) * D;
      }
      *reinterpret_cast<bf16x4*>((PREFILL ? pa.out : da.out) + off + d) = o;
    }
    return;
  }

  if constexpr (!PREFILL) {
    const DecodeArgs& a = da;
    // split partials: (m, l, O) in fp32; row h, split s at prow0 + h * n_splits + s
    const size_t prow0 = ((size_t)b * a.n_q + head0) * a.n_splits;
    auto publish = [&](bool coherent) {
      for (int idx = tid; idx < nrows * D4; idx += NT) {
        const int h = idx / D4;
        const int d = 4 * (idx - h * D4);
        const f32x4 v = red_sum(h, d);
        float* dst = a.part_o + (prow0 + (size_t)h * a.n_splits + split) * D + d;
        if (coherent)
          st16_coherent(dst, v);
        else
          *reinterpret_cast<f32x4*>(dst) = v;
      }
      if (tid < nrows) {
        float* ml = a.part_ml + (prow0 + (size_t)tid * a.n_splits + split) * 2;
        const float lval = n_keys > 0 ? hL[tid] : 0.f;
        if (coherent) {
          st_coherent(ml, hM[tid]);
          st_coherent(ml + 1, lval);
        } else {
          ml[0] = hM[tid];
          ml[1] = lval;
        }
      }
    };
    if (!a.merge_in_kernel) {  // merge_kernel follows
      publish(true);  // written through: less for the end-of-kernel write-back
      return;
    }
    // In-kernel merge: every split publishes its partial, waits for the
    // stores to complete and takes an arrival ticket; the last to arrive
    // merges (its own partial is still in LDS)
    publish(true);
    wait_vmem();
    const size_t grp = ((size_t)b * a.n_kv + g) * a.n_hblk + hblk;
    if (!arrive_last(a.counters + grp, n_used, &s_flag)) return;
    // out = sum_s w_s O_s / sum_s w_s l_s, w_s = 2^(m_s - max m), splits in
    // index order (the result does not depend on which split arrived last);
    // kBatch splits per memory round trip, rescaled between batches.  (A
    // batch of 8, whose loads past the last split repeat the batch's first
    // slot, measured slower on the two-split sliding layers: 25.5 against
    // 25.2 us.  In-kernel merges hold at most kMaxInKernelSplits splits.)
    constexpr int kBatch = 2;
    for (int idx = tid; idx < nrows * D4; idx += NT) {
      const int r = idx / D4;
      const int d = 4 * (idx - r * D4);
      const size_t prow = prow0 + (size_t)r * a.n_splits;
      float M = kNegInf, lsum = 0.f;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < n_used; s0 += kBatch) {
        f32x4 v[kBatch];
        float mv[kBatch], lv[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          // unconditional loads (all in flight at once); past the last split
          // the batch's first one is read again and ignored, and the own
          // split's slot is replaced below
          const int s = s0 + i < n_used ? s0 + i : s0;
          const uint64_t ml = ld8_coherent(a.part_ml + (prow + s) * 2);
          const float* po = a.part_o + (prow + s) * D + d;
          const uint64_t o0 = ld8_coherent(po), o1 = ld8_coherent(po + 2);
          mv[i] = __builtin_bit_cast(float, (uint32_t)ml);
          lv[i] = __builtin_bit_cast(float, (uint32_t)(ml >> 32));
          v[i] = f32x4{__builtin_bit_cast(float, (uint32_t)o0),
                       __builtin_bit_cast(float, (uint32_t)(o0 >> 32)),
                       __builtin_bit_cast(float, (uint32_t)o1),
                       __builtin_bit_cast(float, (uint32_t)(o1 >> 32))};
        }
        if (split >= s0 && split < s0 + kBatch) {
          const int i = split - s0;
          mv[i] = hM[r];
          lv[i] = n_keys > 0 ? hL[r] : 0.f;
          v[i] = red_sum(r, d);
        }
        float bm = M;
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          if (s0 + i < n_used && lv[i] > 0.f) bm = fmaxf(bm, mv[i]);
        if (bm != M) {
          const float sc = fast_exp2(M - bm);  // 0 while nothing was added
          acc *= sc;
          lsum *= sc;
          M = bm;
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          if (s0 + i < n_used && lv[i] > 0.f) {  // empty splits may hold stale data
            const float wt = fast_exp2(mv[i] - M);
            acc += wt * v[i];
            lsum += wt * lv[i];
          }
      }
      const float il = lsum > 0.f ? 1.f / lsum : 0.f;
      bf16x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = (__bf16)(acc[j] * il);
      *reinterpret_cast<bf16x4*>(a.out + ((size_t)b * a.n_q + head0 + r) * D + d) = o;
    }
    if (tid == 0)  // every split of the group has arrived: ready for the next call
      __hip_atomic_store(a.counters + grp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// one attend_kernel launch, with or without the logit cap
template <int D, bool KEQV, int NW, bool PREFILL, bool PAGED, bool NTL, bool FUSED = false>
void attend_launch(bool cap, dim3 grid, hipStream_t s, const DecodeArgs& da,
                   const PrefillArgs& pa) {
  if (cap)
    hipLaunchKernelGGL((attend_kernel<D, KEQV, NW, PREFILL, PAGED, true, NTL, FUSED>), grid,
                       dim3(NW * 64), 0, s, da, pa);
  else
    hipLaunchKernelGGL((attend_kernel<D, KEQV, NW, PREFILL, PAGED, false, NTL, FUSED>), grid,
                       dim3(NW * 64), 0, s, da, pa);
}

template <int D, bool KEQV, bool FUSED>
void decode_launch_as(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  PrefillArgs none{};
  const bool cap = a.softcap != 0;
  if (a.pt.table) {
    if (a.stream_loads)
      attend_launch<D, KEQV, 4, false, true, true, FUSED>(cap, grid, s, a, none);
    else
      attend_launch<D, KEQV, 4, false, true, false, FUSED>(cap, grid, s, a, none);
  } else {
    if (a.stream_loads)
      attend_launch<D, KEQV, 4, false, false, true, FUSED>(cap, grid, s, a, none);
    else
      attend_launch<D, KEQV, 4, false, false, false, FUSED>(cap, grid, s, a, none);
  }
}

template <int D, bool KEQV>
hipError_t decode_launch(const DecodeArgs& a, int batch, hipStream_t s) {
  dim3 grid(a.n_splits, a.n_kv * a.n_hblk, batch);
  if (a.k_new)
    decode_launch_as<D, KEQV, true>(a, grid, s);
  else
    decode_launch_as<D, KEQV, false>(a, grid, s);
  return hipGetLastError();
}

template <int D, bool KEQV>
hipError_t prefill_launch(const PrefillArgs& a, hipStream_t s) {
  // eight waves per row block, four where a wave needs all 512 registers
  // (head_dim 512 with a V plane)
  constexpr int NW = (D >= 512 && !KEQV) ? 4 : 8;
  const int n_log = a.n_rowblk * a.n_kv * a.batch;
  dim3 grid(8 * ((n_log + 7) / 8));
  DecodeArgs none{};
  if (a.pt.table)
    attend_launch<D, KEQV, NW, true, true, false>(a.softcap != 0, grid, s, none, a);
  else
    attend_launch<D, KEQV, NW, true, false, false>(a.softcap != 0, grid, s, none, a);
  return hipGetLastError();
}

}  // namespace

// ---------------------------------------------------------------------------
// library-owned decode scratch (the allocation-free decode entry point)
// ---------------------------------------------------------------------------
//
// Split partials and arrival counters of g4attn_decode_noalloc live here
// instead of in a caller-bound workspace.  Each GPU the library runs on holds
// its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: kernels get the device address that
// hipGetSymbolAddress returns for the current device.

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ __launch_bounds__(256) void zero_kernel(int32_t* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];
}  // namespace

hipError_t scratch_address(void** ptr, bool* first_use) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  *first_use = g_scratch_ptr[dev] == nullptr;
  if (*first_use) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_zero(int32_t* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, int batch, hipStream_t s) {
  dim3 grid(a.n_new * a.n_kv, batch);
  hipLaunchKernelGGL(append_kernel, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t merge_launch(const MergeArgs& a, hipStream_t s) {
  constexpr int D4 = D / 4;
  constexpr int NT = D4 > 64 ? D4 : 64;
  constexpr int R = NT / D4;
  hipLaunchKernelGGL((merge_kernel<D>), dim3((a.rows + R - 1) / R), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  switch (a.D) {
    case 32: return merge_launch<32>(a, s);
    case 64: return merge_launch<64>(a, s);
    case 128: return merge_launch<128>(a, s);
    case 256: return merge_launch<256>(a, s);
    case 512: return merge_launch<512>(a, s);
    default: return hipErrorInvalidValue;
  }
}

#define G4_DISPATCH(FN, ARGS)                                             \
  switch (head_dim) {                                                     \
    case 32: return k_eq_v ? FN<32, true>(ARGS) : FN<32, false>(ARGS);    \
    case 64: return k_eq_v ? FN<64, true>(ARGS) : FN<64, false>(ARGS);    \
    case 128: return k_eq_v ? FN<128, true>(ARGS) : FN<128, false>(ARGS); \
    case 256: return k_eq_v ? FN<256, true>(ARGS) : FN<256, false>(ARGS); \
    case 512: return k_eq_v ? FN<512, true>(ARGS) : FN<512, false>(ARGS); \
    default: return hipErrorInvalidValue;                                 \
  }

hipError_t launch_decode(int head_dim, bool k_eq_v, const DecodeArgs& a, int batch,
                         hipStream_t s) {
#define G4_ARGS a, batch, s
  G4_DISPATCH(decode_launch, G4_ARGS)
#undef G4_ARGS
}

hipError_t launch_prefill(int head_dim, bool k_eq_v, const PrefillArgs& a, hipStream_t s) {
#define G4_ARGS a, s
  G4_DISPATCH(prefill_launch, G4_ARGS)
#undef G4_ARGS
}

}  // namespace g4
