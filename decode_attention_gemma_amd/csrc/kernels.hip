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

#include "internal.h"

namespace g4 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                    __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ __bf16 as_bf16(uint16_t x) { return __builtin_bit_cast(__bf16, x); }

// Split partial results cross workgroups that may run on different XCDs
// (each with its own L2).  They are written and read with the agent-scope
// coherence bit (sc1: write-through / read-around the XCD's L2), the same
// access the compiler emits for agent-scope atomics, and the writer waits for
// the stores to complete before it signals arrival with an agent-scope atomic.
// This avoids the whole-L2 write-back a release fence performs.
__device__ __forceinline__ void st16_coherent(float* p, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}

__device__ __forceinline__ f32x4 ld16_coherent_nowait(const float* p) {
  f32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off sc1" : "=v"(v) : "v"(p) : "memory");
  return v;
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  const int slot = pos % a.cap;
  const int D = a.D;
  const size_t src = ((size_t)(b * a.n_new + t) * a.n_kv + g) * D;
  const size_t seg = (size_t)(b * a.n_kv + g) * a.cap * D;  // elements
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

__device__ __forceinline__ void ld8_coherent_nowait(const float* p, float& a, float& b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 v;
  asm volatile("global_load_dwordx2 %0, %1, off sc1" : "=v"(v) : "v"(p) : "memory");
  a = v[0];
  b = v[1];
}

// In-kernel version, run by the last workgroup of a group to arrive.  All
// (m, l) pairs are fetched in one batch, then the partial outputs in batches
// of up to 8 splits per thread, so the merge costs a few memory round trips.
// `ml` is LDS scratch for n_rows * n_splits * 2 floats.
template <int D>
__device__ void merge_rows_coherent(const float* part_o, const float* part_ml, size_t row0_part,
                                    int n_rows, int n_splits, uint16_t* out,
                                    const size_t* out_row_off, float* ml /*LDS*/,
                                    float* inv_l /*LDS*/, int row_stride) {
  // row r's split s lives at (row0_part + r * row_stride + s); n_splits <= row_stride in use
  const int tid = threadIdx.x;
  const int n_pairs = n_rows * n_splits;
  {
    constexpr int PER = 4;
    float mv[PER], lv[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * (int)blockDim.x;
      const size_t src = row0_part + (size_t)(idx / n_splits) * row_stride + idx % n_splits;
      if (idx < n_pairs) ld8_coherent_nowait(part_ml + src * 2, mv[i], lv[i]);
    }
    wait_vmem();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * (int)blockDim.x;
      if (idx < n_pairs) {
        ml[2 * idx] = mv[i];
        ml[2 * idx + 1] = lv[i];
      }
    }
    for (int idx = tid + PER * (int)blockDim.x; idx < n_pairs; idx += blockDim.x) {
      const size_t src = row0_part + (size_t)(idx / n_splits) * row_stride + idx % n_splits;
      ml[2 * idx] = ld_coherent(part_ml + src * 2);
      ml[2 * idx + 1] = ld_coherent(part_ml + src * 2 + 1);
    }
  }
  __syncthreads();
  // weights in place of m: w_s = 2^(m_s - max m) over splits with l_s > 0
  for (int r = tid; r < n_rows; r += blockDim.x) {
    float* p = ml + 2 * r * n_splits;
    float M = kNegInf;
    for (int s = 0; s < n_splits; ++s)
      if (p[2 * s + 1] > 0.f) M = fmaxf(M, p[2 * s]);
    float lsum = 0.f;
    for (int s = 0; s < n_splits; ++s) {
      const float l = p[2 * s + 1];
      const float w = l > 0.f ? fast_exp2(p[2 * s] - M) : 0.f;
      p[2 * s] = w;
      lsum += w * l;
    }
    inv_l[r] = lsum > 0.f ? 1.f / lsum : 0.f;
  }
  __syncthreads();
  constexpr int D4 = D / 4;
  constexpr int BATCH = 8;
  for (int idx = tid; idx < n_rows * D4; idx += blockDim.x) {
    const int r = idx / D4;
    const int d = 4 * (idx - r * D4);
    const float* po = part_o + (row0_part + (size_t)r * row_stride) * D + d;
    const float* wr = ml + 2 * r * n_splits;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n_splits; s0 += BATCH) {
      f32x4 v[BATCH];
#pragma unroll
      for (int i = 0; i < BATCH; ++i)
        if (s0 + i < n_splits) v[i] = ld16_coherent_nowait(po + (size_t)(s0 + i) * D);
      wait_vmem();
#pragma unroll
      for (int i = 0; i < BATCH; ++i)
        if (s0 + i < n_splits) {
          const float w = wr[2 * (s0 + i)];
          if (w != 0.f) acc += w * v[i];  // empty splits hold stale data: skip them
        }
    }
    const float il = inv_l[r];
    bf16x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = (__bf16)(acc[j] * il);
    *reinterpret_cast<bf16x4*>(out + out_row_off[r] + d) = o;
  }
}

// Stand-alone version: one workgroup per output row; partials are ordinary
// global memory here (a kernel boundary separates writer and reader).
__global__ __launch_bounds__(128) void merge_kernel(MergeArgs a) {
  __shared__ float wgt[kMaxDecodeSplits];
  __shared__ float s_inv;
  const size_t row = blockIdx.x;
  size_t out_off = row * a.D;
  if (a.prefill) {
    const int grp = (int)(row / a.rows_per_group);
    const int r = (int)(row - (size_t)grp * a.rows_per_group);
    const int b = grp / a.n_kv, g = grp - (grp / a.n_kv) * a.n_kv;
    const int t = r / a.G, h = r - (r / a.G) * a.G;
    out_off = (((size_t)b * a.T + t) * a.n_q + g * a.G + h) * a.D;
  }
  int n_used = a.n_splits;
  if (!a.prefill) {
    const int bseq = (int)(row / a.n_q);
    int L = a.seq_lens[bseq];
    L = L < 0 ? 0 : (L > a.kv_max ? a.kv_max : L);
    const int lo = a.window > 0 ? max(0, L - a.window) : 0;
    int f, e;
    decode_split_range(lo, L, a.KB, a.blocks_per_split, 0, &n_used, &f, &e);
    if (n_used <= 1) return;  // written by the decode kernel itself
  }
  const float* ml = a.part_ml + row * a.n_splits * 2;
  // every thread of the first wave takes one split; a wave-wide max/sum
  if (threadIdx.x < 64) {
    const int s = threadIdx.x;
    const bool ok = s < n_used;
    const float m = ok ? ml[2 * s] : kNegInf;
    const float l = ok ? ml[2 * s + 1] : 0.f;
    float M = l > 0.f ? m : kNegInf;
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float w = l > 0.f ? fast_exp2(m - M) : 0.f;
    float lsum = w * l;
    for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);
    if (ok) wgt[s] = w;
    if (s == 0) s_inv = lsum > 0.f ? 1.f / lsum : 0.f;
  }
  __syncthreads();
  const float* po = a.part_o + row * a.n_splits * a.D;
  constexpr int BATCH = 8;
  for (int d = 4 * threadIdx.x; d < a.D; d += 4 * blockDim.x) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n_used; s0 += BATCH) {
      f32x4 v[BATCH];
#pragma unroll
      for (int i = 0; i < BATCH; ++i)
        if (s0 + i < n_used)
          v[i] = *reinterpret_cast<const f32x4*>(po + (size_t)(s0 + i) * a.D + d);
#pragma unroll
      for (int i = 0; i < BATCH; ++i)
        if (s0 + i < n_used && wgt[s0 + i] != 0.f) acc += wgt[s0 + i] * v[i];
    }
    bf16x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = (__bf16)(acc[j] * s_inv);
    *reinterpret_cast<bf16x4*>(a.out + out_off + d) = o;
  }
}

// ---------------------------------------------------------------------------
// decode: one workgroup per (key split, KV head x head block, sequence)
// ---------------------------------------------------------------------------
//
// The workgroup's key range is cut into blocks of KB keys (32, or 16 on k_eq_v
// layers), and wave w takes blocks w, w+4, ...: each wave streams its blocks
// straight from HBM into registers in operand order (1 KiB contiguous per load
// instruction), keeps its own online-softmax state, and needs no barrier until
// the four waves combine their states through LDS at the end.  Latency is
// hidden by occupancy (several independent waves per SIMD) rather than by a
// shared pipeline.  On k_eq_v layers the K block is the V block as well; it is
// written once to a wave-private LDS area and read back transposed.

template <int D, bool KEQV>
struct DecodeShape {
  static constexpr int KB = KEQV ? 16 : 32;  // keys per block
  static constexpr int NSB = KB / 16;        // 16-key score blocks per block
  static constexpr int KS = D / 32;          // 1 KiB K sub-tiles per 16 keys
  static constexpr int NDB = D / 16;         // 16-dim output blocks
  static constexpr int RED_FLOATS = 16 * D;  // cross-wave reduction buffer
  static constexpr int TR_ELEMS = KEQV ? 16 * D : 0;  // per-wave transpose area
  static constexpr int MERGE_BYTES = (2 * 16 * kMaxDecodeSplits + 16) * 4;
  static constexpr int A_BYTES = (4 * TR_ELEMS * 2 > RED_FLOATS * 4) ? 4 * TR_ELEMS * 2 : RED_FLOATS * 4;
  static constexpr int LDS_BYTES = A_BYTES > MERGE_BYTES ? A_BYTES : MERGE_BYTES;
};

template <int D, bool KEQV>
__global__ __launch_bounds__(256, D >= 512 ? 1 : 2) void decode_kernel(DecodeArgs a) {
  using S = DecodeShape<D, KEQV>;
  constexpr int KB = S::KB, NSB = S::NSB, KS = S::KS, NDB = S::NDB;
  constexpr int D4 = D / 4;

  __shared__ __attribute__((aligned(16))) unsigned char lds[S::LDS_BYTES];
  __shared__ float wm[4][16], wl[4][16], hM[16], hL[16];
  __shared__ int s_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int c16 = lane & 15;
  const int q4 = lane >> 4;
  const int split = blockIdx.x;
  const int g = blockIdx.y / a.n_hblk;
  const int hblk = blockIdx.y - g * a.n_hblk;
  const int b = blockIdx.z;
  const int head0 = g * a.G + hblk * 16;
  const int nh = min(16, a.G - hblk * 16);

  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.kv_max ? a.kv_max : L);
  const int lo = a.window > 0 ? max(0, L - a.window) : 0;
  // the sequence's KB-aligned blocks are dealt out evenly to the splits it
  // uses; the number it uses grows with its length
  int n_used, blk_first, blk_end;
  decode_split_range(lo, L, KB, a.blocks_per_split, split, &n_used, &blk_first, &blk_end);
  if (split > 0 && split >= n_used) return;  // nothing for this workgroup
  const bool direct = n_used <= 1;           // write the output, no partials
  const int r_beg = max(lo, blk_first * KB);
  const int r_end = min(L, blk_end * KB);
  const int n_keys = r_end - r_beg;

  const size_t seg = (size_t)(b * a.n_kv + g) * a.cap * D;
  const uint16_t* kseg = a.kp + seg;
  const uint16_t* vseg = a.vp + seg;

  // loads of a wave's next block are issued as soon as the registers they
  // land in are free (K after the scores, V after the PV product), so they
  // overlap the rest of the current block
  u32x4 kreg[NSB][KS];
  u32x4 vreg[KEQV ? 1 : NDB];
  auto load_k = [&](int blk) {
    const int slot0 = (blk * KB) % a.cap;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        kreg[sb][s] = ldg16(kseg + ((size_t)(slot0 / 16 + sb) * KS + s) * 512 + lane * 8);
  };
  auto load_v = [&](int blk) {
    if constexpr (!KEQV) {
      const int slot0 = (blk * KB) % a.cap;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        vreg[db] = ldg16(vseg + ((size_t)(slot0 / 32) * NDB + db) * 512 + lane * 8);
    }
  };
  if (n_keys > 0 && blk_first + w < blk_end) {
    load_k(blk_first + w);
    load_v(blk_first + w);
  }

  // queries as the B operand of S^T = K Q^T (column c16 = head, k-slots =
  // dims), kept in LDS in operand order: sub-tile s, lane L at (s*64 + L)*8
  __shared__ __attribute__((aligned(16))) uint16_t Qs[KS * 512];
  {
    const uint16_t* qrow = a.q + ((size_t)b * a.n_q + head0 + c16) * D + 8 * q4;
    for (int s = w; s < KS; s += 4)
      *reinterpret_cast<u32x4*>(&Qs[(s * 64 + lane) * 8]) =
          c16 < nh ? ldg16(qrow + 32 * s) : u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  f32x4 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;
  float l_run = 0.f;

  uint16_t* tr = reinterpret_cast<uint16_t*>(lds) + w * S::TR_ELEMS;  // k_eq_v only

  if (n_keys > 0) {
    for (int blk = blk_first + w; blk < blk_end; blk += 4) {
      const int pos0 = blk * KB;
      const bool has_next = blk + 4 < blk_end;
      const bool full = pos0 >= r_beg && pos0 + KB <= r_end;

      // scores, mask, online softmax (lane's column c16 = head).  The compiler
      // barrier keeps the query reads from LDS here instead of hoisting the
      // whole query operand into registers for the loop.
      asm volatile("" ::: "memory");
      f32x4 sacc[NSB];
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        sacc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 qf = *reinterpret_cast<const bf16x8*>(&Qs[(s * 64 + lane) * 8]);
          sacc[sb] = mfma32(as_bf16x8(kreg[sb][s]), qf, sacc[sb]);
        }
      }
      if constexpr (KEQV) {
        // the K block doubles as V: stage it in this wave's LDS area in its
        // operand order, to be read back transposed
#pragma unroll
        for (int s = 0; s < KS; ++s)
          *reinterpret_cast<u32x4*>(tr + s * 512 + lane * 8) = kreg[0][s];
      }
      if (has_next) load_k(blk + 4);
      float lmax = kNegInf;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kpos = pos0 + 16 * sb + 4 * q4 + j;
          const bool ok = full || (kpos >= r_beg && kpos < r_end);
          sacc[sb][j] = ok ? sacc[sb][j] * a.scale_log2 : kNegInf;
          lmax = fmaxf(lmax, sacc[sb][j]);
        }
      }
      lmax = fmaxf(lmax, __shfl_xor(lmax, 16));
      lmax = fmaxf(lmax, __shfl_xor(lmax, 32));
      const float m_new = fmaxf(m_run, lmax);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
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
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;

      if constexpr (!KEQV) {
        // P^T as the B operand: k-slot j <-> key 4q+j (j<4) / 16+4q+j-4
        bf16x8 pf;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pf[j] = pb[0][j];
          pf[4 + j] = pb[1][j];
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          bf16x8 vf = as_bf16x8(vreg[db]);
          if (!full) {  // values of keys outside the range must not reach the MFMA
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int kk = (j < 4) ? 4 * q4 + j : 16 + 4 * q4 + j - 4;
              const int kpos = pos0 + kk;
              if (kpos < r_beg || kpos >= r_end) vf[j] = (__bf16)0.f;
            }
          }
          oacc[db] = mfma32(vf, pf, oacc[db]);
        }
        if (has_next) load_v(blk + 4);
      } else {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = 16 * db + c16;
          const uint16_t* col = tr + (d / 32) * 512 + ((d % 32) / 8) * 128 + (d % 8);
          bf16x4 vf;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int kk = 4 * q4 + j;
            vf[j] = as_bf16(col[kk * 8]);
            if (!full) {
              const int kpos = pos0 + kk;
              if (kpos < r_beg || kpos >= r_end) vf[j] = (__bf16)0.f;
            }
          }
          oacc[db] = mfma16(vf, pb[0], oacc[db]);
        }
      }
    }
  }

  // ---- combine the four waves: common max, rescale, sum through LDS ----
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
  for (int i = 0; i < 4; ++i) M = fmaxf(M, wm[i][c16]);
  const float M_use = M == kNegInf ? 0.f : M;
  if (tid < 16) {
    float Lh = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) Lh += wl[i][tid] * fast_exp2(wm[i][tid] - M_use);
    hM[tid] = M;
    hL[tid] = Lh;
  }
  const float mine = fast_exp2(m_run - M_use);
  float* red = reinterpret_cast<float*>(lds);  // [16][D]
  for (int step = 3; step >= 0; --step) {
    if (w == step && c16 < nh) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        float* p = red + c16 * D + 16 * db + 4 * q4;
        f32x4 v = oacc[db] * mine;
        if (step != 3) v += *reinterpret_cast<f32x4*>(p);
        *reinterpret_cast<f32x4*>(p) = v;
      }
    }
    __syncthreads();
  }

  // red[h][:] = unnormalised O of this key range for head h; hM, hL per head
  if (direct) {
    for (int idx = tid; idx < nh * D4; idx += 256) {
      const int h = idx / D4;
      const int d = 4 * (idx - h * D4);
      const float il = hL[h] > 0.f ? 1.f / hL[h] : 0.f;
      const f32x4 v = *reinterpret_cast<const f32x4*>(red + h * D + d);
      bf16x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = (__bf16)(v[j] * il);
      *reinterpret_cast<bf16x4*>(a.out + ((size_t)b * a.n_q + head0 + h) * D + d) = o;
    }
    return;
  }

  // split partial: (m, l, O) in fp32
  const size_t prow0 = ((size_t)b * a.n_q + head0) * a.n_splits + split;
  for (int idx = tid; idx < nh * D4; idx += 256) {
    const int h = idx / D4;
    const int d = 4 * (idx - h * D4);
    const f32x4 v = *reinterpret_cast<const f32x4*>(red + h * D + d);
    float* dst = a.part_o + (prow0 + (size_t)h * a.n_splits) * D + d;
    if (a.merge_in_kernel)
      st16_coherent(dst, v);
    else
      *reinterpret_cast<f32x4*>(dst) = v;
  }
  if (tid < nh) {
    float* ml = a.part_ml + (prow0 + (size_t)tid * a.n_splits) * 2;
    const float lval = n_keys > 0 ? hL[tid] : 0.f;
    if (a.merge_in_kernel) {
      st_coherent(ml, hM[tid]);
      st_coherent(ml + 1, lval);
    } else {
      ml[0] = hM[tid];
      ml[1] = lval;
    }
  }
  if (!a.merge_in_kernel) return;
  wait_vmem();
  int32_t* ctr = a.counters + ((size_t)b * a.n_kv + g) * a.n_hblk + hblk;
  if (!arrive_last(ctr, n_used, &s_flag)) return;

  float* wgt = reinterpret_cast<float*>(lds);  // 16 x n_splits (m, l) pairs
  float* inv_l = wgt + 2 * 16 * kMaxDecodeSplits;
  __shared__ size_t out_off[16];
  if (tid < nh) out_off[tid] = ((size_t)b * a.n_q + head0 + tid) * D;
  __syncthreads();
  merge_rows_coherent<D>(a.part_o, a.part_ml, ((size_t)b * a.n_q + head0) * a.n_splits, nh,
                         n_used, a.out, out_off, wgt, inv_l, a.n_splits);
  if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// prefill: one workgroup per (key split, 64-row block, sequence x KV head)
// ---------------------------------------------------------------------------
//
// Rows of a (sequence, KV head) group are the T x G (token, head) pairs,
// token-major.  Wave w owns 16 rows: it keeps their queries as MFMA operands
// in registers and their output O^T in accumulators; the four waves share the
// K/V tiles, copied verbatim (operand-ordered) from the cache into LDS, so
// every operand read from LDS is a conflict-free 16 bytes per lane.

template <int D, bool KEQV, int KT>
__global__ __launch_bounds__(256, 1) void prefill_kernel(PrefillArgs a) {
  constexpr int KS = D / 32;
  constexpr int NDB = D / 16;
  constexpr int NKB = KT / 16;              // 16-key score blocks per tile
  constexpr int K_ELEMS = KT * D;           // K tile (operand order)
  constexpr int V_ELEMS = KEQV ? 0 : KT * D;
  constexpr int CH_TILE = K_ELEMS / 8;      // 16-byte chunks per plane tile
  constexpr int CH_THR = (CH_TILE + 255) / 256;

  // the K tile's space also serves the split merge: (m, l) per row and split
  constexpr int MERGE_ELEMS = 2 * (2 * kPrefillRows * kMaxPrefillSplits + kPrefillRows);
  __shared__ __attribute__((aligned(16))) uint16_t Ks[K_ELEMS > MERGE_ELEMS ? K_ELEMS : MERGE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[KEQV ? 8 : V_ELEMS];
  __shared__ int s_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int c16 = lane & 15;
  const int q4 = lane >> 4;
  const int split = blockIdx.x;
  const int rowblk = blockIdx.y;
  const int b = blockIdx.z / a.n_kv;
  const int g = blockIdx.z - b * a.n_kv;

  int start = a.start_pos[b];
  start = start < 0 ? 0 : start;
  const int rowbase = rowblk * kPrefillRows;
  const int last_row = min(a.rows, rowbase + kPrefillRows) - 1;
  const int p_first = start + rowbase / a.G;
  const int p_last = start + last_row / a.G;
  const int kbeg = a.window > 0 ? max(0, p_first - a.window + 1) : 0;
  const int kend = min(p_last + 1, a.kv_max);
  const int base = kbeg & ~(KT - 1);  // splits and tiles aligned to KT positions
  const int r_beg = max(kbeg, base + split * a.split_keys);
  const int r_end = min(kend, base + (split + 1) * a.split_keys);
  const int n_keys = r_end - r_beg;

  const int row = rowbase + 16 * w + c16;
  const bool row_ok = row < a.rows;
  const int t_row = row_ok ? row / a.G : 0;
  const int h_row = row_ok ? row - t_row * a.G : 0;
  const int p_row = start + t_row;
  const int lo_row = a.window > 0 ? max(0, p_row - a.window + 1) : 0;
  const int wr0 = min(rowbase + 16 * w, a.rows - 1);
  const int wr1 = min(rowbase + 16 * w + 15, a.rows - 1);
  const bool wave_has_rows = rowbase + 16 * w < a.rows;
  const int w_lo = a.window > 0 ? max(0, start + wr0 / a.G - a.window + 1) : 0;
  const int w_hi = start + wr1 / a.G + 1;

  const size_t seg = (size_t)(b * a.n_kv + g) * a.cap * D;
  const uint16_t* kseg = a.kp + seg;
  const uint16_t* vseg = a.vp + seg;

  bf16x8 qf[KS];
  {
    const uint16_t* qrow =
        a.q + (((size_t)b * a.T + t_row) * a.n_q + g * a.G + h_row) * D + 8 * q4;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = row_ok ? as_bf16x8(ldg16(qrow + 32 * s)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }

  f32x4 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;
  float l_run = 0.f;

  // a tile is KT consecutive positions starting at a multiple of KT; in the
  // cache it is one contiguous run of K_ELEMS (and V_ELEMS) elements
  u32x4 kreg[CH_THR];
  u32x4 vreg[KEQV ? 1 : CH_THR];
  auto load_tile = [&](int tpos) {
    const size_t off = (size_t)(tpos % a.cap) * D;
#pragma unroll
    for (int i = 0; i < CH_THR; ++i) {
      const int c = tid + 256 * i;
      if (c < CH_TILE) {
        kreg[i] = ldg16(kseg + off + 8 * c);
        if constexpr (!KEQV) vreg[i] = ldg16(vseg + off + 8 * c);
      }
    }
  };

  const int t_first = n_keys > 0 ? r_beg / KT : 0;
  const int t_end = n_keys > 0 ? (r_end + KT - 1) / KT : 0;
  if (t_end > t_first) load_tile(t_first * KT);

  for (int t = t_first; t < t_end; ++t) {
    const int tpos = t * KT;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CH_THR; ++i) {
      const int c = tid + 256 * i;
      if (c < CH_TILE) {
        *reinterpret_cast<u32x4*>(&Ks[8 * c]) = kreg[i];
        if constexpr (!KEQV) *reinterpret_cast<u32x4*>(&Vs[8 * c]) = vreg[i];
      }
    }
    __syncthreads();
    if (t + 1 < t_end) load_tile(tpos + KT);

    const int vis_lo_t = max(r_beg, tpos);
    const int vis_hi_t = min(r_end, tpos + KT);
    if (!wave_has_rows || vis_lo_t >= w_hi || vis_hi_t <= w_lo) continue;
    const bool tile_full = vis_lo_t == tpos && vis_hi_t == tpos + KT;

    f32x4 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&Ks[(kb * KS + s) * 512 + lane * 8]);
        sacc[kb] = mfma32(kf, qf[s], sacc[kb]);
      }
    }
    const int vis_lo = max(lo_row, vis_lo_t);
    const int vis_hi = min(p_row + 1, vis_hi_t);
    float lmax = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kpos = tpos + 16 * kb + 4 * q4 + j;
        const bool ok = row_ok && kpos >= vis_lo && kpos < vis_hi;
        sacc[kb][j] = ok ? sacc[kb][j] * a.scale_log2 : kNegInf;
        lmax = fmaxf(lmax, sacc[kb][j]);
      }
    }
    lmax = fmaxf(lmax, __shfl_xor(lmax, 16));
    lmax = fmaxf(lmax, __shfl_xor(lmax, 32));
    const float m_new = fmaxf(m_run, lmax);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
    bf16x4 pb[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const __bf16 p = (__bf16)fast_exp2(sacc[kb][j] - m_use);
        pb[kb][j] = p;
        psum += (float)p;
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;

#pragma unroll
    for (int kk = 0; kk < NKB / 2; ++kk) {
      bf16x8 pf;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pf[j] = pb[2 * kk][j];
        pf[4 + j] = pb[2 * kk + 1][j];
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        bf16x8 vf;
        if constexpr (!KEQV) {
          vf = *reinterpret_cast<const bf16x8*>(&Vs[(kk * NDB + db) * 512 + lane * 8]);
        } else {
          // V^T from the operand-ordered K tile: key kslot(q, j), dim d
          const int d = 16 * db + c16;
          const uint16_t* col = &Ks[(d / 32) * 512 + ((d % 32) / 8) * 128 + (d % 8)];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            vf[j] = as_bf16(col[((2 * kk) * KS) * 512 + (4 * q4 + j) * 8]);
            vf[4 + j] = as_bf16(col[((2 * kk + 1) * KS) * 512 + (4 * q4 + j) * 8]);
          }
        }
        if (!tile_full) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int kkey = 32 * kk + ((j < 4) ? 4 * q4 + j : 16 + 4 * q4 + j - 4);
            const int kpos = tpos + kkey;
            if (kpos < vis_lo_t || kpos >= vis_hi_t) vf[j] = (__bf16)0.f;
          }
        }
        oacc[db] = mfma32(vf, pf, oacc[db]);
      }
    }
  }

  float lt = l_run;
  lt += __shfl_xor(lt, 16);
  lt += __shfl_xor(lt, 32);

  if (a.n_splits == 1) {
    if (row_ok) {
      const float il = lt > 0.f ? 1.f / lt : 0.f;
      uint16_t* orow = a.out + (((size_t)b * a.T + t_row) * a.n_q + g * a.G + h_row) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        bf16x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = (__bf16)(oacc[db][j] * il);
        *reinterpret_cast<bf16x4*>(orow + 16 * db + 4 * q4) = o;
      }
    }
    return;
  }

  const size_t grp_row0 = (size_t)(b * a.n_kv + g) * a.rows;
  if (row_ok) {
    const size_t prow = (grp_row0 + row) * a.n_splits + split;
    if (n_keys > 0) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        float* dst = a.part_o + prow * D + 16 * db + 4 * q4;
        if (a.merge_in_kernel)
          st16_coherent(dst, oacc[db]);
        else
          *reinterpret_cast<f32x4*>(dst) = oacc[db];
      }
    }
    if (q4 == 0) {
      if (a.merge_in_kernel) {
        st_coherent(a.part_ml + prow * 2, m_run);
        st_coherent(a.part_ml + prow * 2 + 1, n_keys > 0 ? lt : 0.f);
      } else {
        a.part_ml[prow * 2] = m_run;
        a.part_ml[prow * 2 + 1] = n_keys > 0 ? lt : 0.f;
      }
    }
  }
  if (!a.merge_in_kernel) return;
  wait_vmem();
  int32_t* ctr = a.counters + ((size_t)b * a.n_kv + g) * a.n_rowblk + rowblk;
  if (!arrive_last(ctr, a.n_splits, &s_flag)) return;

  const int n_rows = last_row - rowbase + 1;
  float* wgt = reinterpret_cast<float*>(Ks);  // kPrefillRows x n_splits (m, l) pairs
  float* inv_l = wgt + 2 * kPrefillRows * kMaxPrefillSplits;
  __shared__ size_t out_off[kPrefillRows];
  if (tid < n_rows) {
    const int r = rowbase + tid;
    const int tt = r / a.G;
    const int hh = r - tt * a.G;
    out_off[tid] = (((size_t)b * a.T + tt) * a.n_q + g * a.G + hh) * D;
  }
  __syncthreads();
  merge_rows_coherent<D>(a.part_o, a.part_ml, (grp_row0 + rowbase) * a.n_splits, n_rows,
                         a.n_splits, a.out, out_off, wgt, inv_l, a.n_splits);
  if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, bool KEQV>
hipError_t decode_launch(const DecodeArgs& a, int batch, hipStream_t s) {
  dim3 grid(a.n_splits, a.n_kv * a.n_hblk, batch);
  hipLaunchKernelGGL((decode_kernel<D, KEQV>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, bool KEQV>
hipError_t prefill_launch(const PrefillArgs& a, int batch, hipStream_t s) {
  dim3 grid(a.n_splits, a.n_rowblk, batch * a.n_kv);
  constexpr int KT = D >= 512 ? 32 : 64;
  hipLaunchKernelGGL((prefill_kernel<D, KEQV, KT>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int batch, hipStream_t s) {
  dim3 grid(a.n_new * a.n_kv, batch);
  hipLaunchKernelGGL(append_kernel, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3(a.rows), dim3(128), 0, s, a);
  return hipGetLastError();
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

hipError_t launch_prefill(int head_dim, bool k_eq_v, const PrefillArgs& a, int batch,
                          hipStream_t s) {
#define G4_ARGS a, batch, s
  G4_DISPATCH(prefill_launch, G4_ARGS)
#undef G4_ARGS
}

}  // namespace g4
