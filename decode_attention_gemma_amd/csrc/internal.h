// Internal interfaces between the host plan (plan.cpp) and the HIP kernels
// (kernels.hip).  Not part of the public ABI.
//
// Cache layout (per owning layer, per (sequence, KV head) segment of `cap`
// slots, cap a multiple of 64; position p lives in slot p mod cap):
//
//   K plane: 16-slot blocks; a block holds head_dim/32 sub-tiles of
//            16 keys x 32 dims = 1 KiB, each stored in the lane order of a
//            v_mfma_f32_16x16x32_bf16 operand: lane L = key + 16 q holds
//            dims 8q .. 8q+7 of its sub-tile's 32 (16 bytes per lane).
//   V plane: 32-slot blocks; a block holds head_dim/16 sub-tiles of
//            32 keys x 16 dims = 1 KiB, lane L = dim + 16 q holding the keys
//            4q .. 4q+3 and 16+4q .. 16+4q+3 of the block (16 bytes per lane),
//            i.e. V^T already in operand order for O^T += V^T P^T.
//
// so that every cache read of the kernels is a contiguous 1 KiB per wave
// instruction.  k_eq_v layers have only the K plane.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace g4 {

// Upper bound on decode key splits per (sequence, head block).
constexpr int kMaxDecodeSplits = 64;
// Query rows (token x head pairs) per prefill workgroup.
constexpr int kPrefillRows = 16;

// Keys per decode key block, on layers with and without a V plane.
constexpr int kDecodeBlock = 32;
// A decode call that reads more cache bytes than this streams them past the
// caches (non-temporal loads): more than the eight XCDs' L2s hold together.
// Smaller calls use the default policy, so that a small cache stays resident
// from one step to the next.
constexpr int64_t kStreamLoadBytes = int64_t(32) << 20;

// Waves per SIMD an attention kernel instance is built for: 2 (up to 256
// registers per lane), or 1 where one wave needs more (head_dim 512 without
// k_eq_v: its V block and accumulators alone take 256) or where the LDS
// admits one workgroup per CU anyway (head_dim 512 decode, whose combine
// takes a reduction slot per wave).  (Deeper per-wave prefetch at one wave
// per SIMD measured slower on every layer type: with a single wave per SIMD
// nothing hides its own latencies.)
__host__ __device__ constexpr int waves_per_simd(int head_dim, bool k_eq_v, bool prefill) {
  return head_dim >= 512 && (!k_eq_v || !prefill) ? 1 : 2;
}

// Byte offsets of element d of the K row / V row in one segment.
__host__ __device__ inline int64_t k_elem_offset(int64_t slot, int d, int D) {
  const int64_t blk = slot / 16, kk = slot % 16;
  return ((blk * (D / 32) + d / 32) * 64 + ((d % 32) / 8) * 16 + kk) * 16 + (d % 8) * 2;
}
__host__ __device__ inline int64_t v_elem_offset(int64_t slot, int d, int D) {
  const int64_t blk = slot / 32;
  const int kk = (int)(slot % 32);
  const int q = (kk % 16) / 4;
  const int j = (kk / 16) * 4 + kk % 4;
  return ((blk * (D / 16) + d / 16) * 64 + q * 16 + d % 16) * 16 + j * 2;
}

// Paged cache: position p of sequence b lives in physical page
// table[b * stride + p / page] at slot p % page.  A page holds `page` slots
// (a multiple of 64) of every KV head of one owning layer: (page, head) is a
// segment of page * D elements in the operand order of an unpaged segment.
// table == nullptr: the unpaged layout (segment (b, head) of cap slots).
struct PageTable {
  const int32_t* table;  // [batch][stride] physical page ids, or nullptr
  int stride;            // entries per sequence (= kv_max / page)
  int page;              // slots per page
  int n_pages;           // pages in each plane; ids are clamped into [0, n_pages)
};

// LDS entries for the page ids a workgroup's key range spans.
constexpr int kMaxWgPages = 1024;

__host__ __device__ inline int clamp_page(int id, int n_pages) {
  return id < 0 ? 0 : (id >= n_pages ? n_pages - 1 : id);
}

struct AppendArgs {
  const uint16_t* k;  // [batch][n_new][n_kv][D]
  const uint16_t* v;  // same, or nullptr when the layer has no V plane
  uint16_t* kp;       // owner K plane
  uint16_t* vp;       // owner V plane, or nullptr
  const int32_t* start;
  const int32_t* nvalid;  // nullable
  int n_new, n_kv, D, cap, kv_max;
  PageTable pt;
};

struct DecodeArgs {
  const uint16_t* q;  // [B][n_q][D]
  uint16_t* kp;       // written only when k_new is set
  uint16_t* vp;       // == kp when k_eq_v
  // Optional: the current token's K (and V) rows [B][n_kv][D], written into
  // the cache at position seq_lens[b] - 1 before it is attended (nullptr:
  // the token is already in the cache)
  const uint16_t* k_new;
  const uint16_t* v_new;  // nullptr when k_eq_v
  const int32_t* seq_lens;
  uint16_t* out;     // [B][n_q][D]
  float* part_o;     // [B][n_q][n_splits][D]
  float* part_ml;    // [B][n_q][n_splits][2]
  int32_t* counters; // [B][n_kv][n_hblk]
  int n_q, n_kv, G, n_hblk, cap, window, kv_max;
  // host bound on seq_lens[b] (<= kv_max) that the split grid is planned
  // from; longer lengths are clamped to it, so a violated bound changes the
  // numbers but never the grid's coverage or the arrival counts
  int max_len;
  // A sequence with nb key blocks uses ceil(nb / blocks_per_split) splits
  // (at most n_splits, the grid's x extent), so every split streams about
  // the same number of blocks whatever the sequence's length.
  int blocks_per_split, n_splits;
  int merge_in_kernel;  // 1: last arriving workgroup merges; 0: a merge kernel follows
  // 1: cache rows are loaded with the non-temporal hint (the call reads more
  // than kStreamLoadBytes); 0: default cache policy
  int stream_loads;
  float scale_log2;     // scale * log2(e)
  // attention-logit cap c (softcap != 0): score * log2(e) =
  // cap_log2 * tanh(q.k * cap_in), cap_in = scale / c, cap_log2 = c * log2(e)
  int softcap;
  float cap_in, cap_log2;
  PageTable pt;
};

// Key blocks [first, end) of split `split` of a sequence whose visible keys
// are [lo, L), and the number of splits the sequence uses.
__host__ __device__ inline void decode_split_range(int lo, int L, int KB, int blocks_per_split,
                                                   int split, int* n_used, int* first,
                                                   int* end) {
  const int nb = L > lo ? (L + KB - 1) / KB - lo / KB : 0;
  const int nu = nb > 0 ? (nb + blocks_per_split - 1) / blocks_per_split : 0;
  *n_used = nu;
  if (split >= nu) {
    *first = *end = 0;
    return;
  }
  *first = lo / KB + (int)(((long long)split * nb) / nu);
  *end = lo / KB + (int)(((long long)(split + 1) * nb) / nu);
}

struct PrefillArgs {
  const uint16_t* q;  // [B][T][n_q][D]
  const uint16_t* kp;
  const uint16_t* vp;  // == kp when k_eq_v
  const int32_t* start_pos;
  uint16_t* out;  // [B][T][n_q][D]
  int batch, n_q, n_kv, G, T, cap, window, kv_max;
  int max_start;  // host bound on start_pos[b]; larger starts are clamped to it
  // rows = T * G (token-major (token, head) pairs of one KV head), in
  // n_rowblk blocks of kPrefillRows
  int rows, n_rowblk;
  float scale_log2;
  int softcap;  // as in DecodeArgs
  float cap_in, cap_log2;
  PageTable pt;
};

struct MergeArgs {
  const float* part_o;   // [rows][n_splits][D], rows = (sequence, query head)
  const float* part_ml;  // [rows][n_splits][2]
  uint16_t* out;         // row r at out[r * D]
  int rows, n_splits, D, n_q;
  // splits in use per row follow from the sequence's length; rows of
  // sequences with at most one split were written by the decode kernel
  const int32_t* seq_lens;
  int window, kv_max, max_len, KB, blocks_per_split;
};

// Library-owned decode scratch (allocation-free decode): kScratchBytes per
// GPU, the first kScratchCounterBytes of it arrival counters.
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr size_t kScratchCounterBytes = size_t(256) << 10;
// Device address of the current GPU's scratch; *first_use is set on the
// first lookup on that GPU (its counters must then be zeroed once).
hipError_t scratch_address(void** ptr, bool* first_use);
hipError_t launch_zero(int32_t* p, int n, hipStream_t s);

hipError_t launch_append(const AppendArgs& a, int batch, hipStream_t s);
hipError_t launch_decode(int head_dim, bool k_eq_v, const DecodeArgs& a, int batch, hipStream_t s);
hipError_t launch_prefill(int head_dim, bool k_eq_v, const PrefillArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);

}  // namespace g4
