// Hardware-rate probes for this GPU, the practical bounds the attention
// kernels are measured against.  Not part of the attention library or its C
// ABI; bench.py --read-probe / --gemm-probe load them from their own shared
// library.
//
// read_kernel: HBM streaming read rate (the decode kernels read each cache
// byte once per call).  Every thread reads 16-byte vectors in a grid-stride
// loop, U of them in flight per iteration, with or without the non-temporal
// hint, and folds them into a value that is stored only if it equals a fixed
// pattern, so the loads cannot be removed.
//
// mfma_kernel: issue rate of back-to-back v_mfma_f32_16x16x32_bf16 with C
// independent accumulation chains per wave, no memory traffic: the matrix
// cores' own ceiling, apart from any operand delivery.
//
// lds_kernel / l2_kernel: per-CU operand delivery, what bounds the prefill
// kernels (their MFMA operands come from LDS, their key blocks from L2): the
// LDS read rate of 16-byte reads and of the transposing 8-byte reads, and the
// L2 -> CU load rate into registers or straight into LDS.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

template <bool NT, int U>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ p, size_t n,
                                                   u32x4* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld<NT>(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= ld<NT>(p + i);
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0x85ebca6bu && acc.w == 0xc2b2ae35u)
    sink[threadIdx.x] = acc;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int C>
__global__ __launch_bounds__(512) void mfma_kernel(int iters, float* sink) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 0.001f + i);
    b[i] = (__bf16)(i * 0.5f);
  }
  f32x4 c[C];
#pragma unroll
  for (int i = 0; i < C; ++i) c[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < C; ++i) c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < C; ++i) s += c[i][0] + c[i][1] + c[i][2] + c[i][3];
  if (s == 1.2345f) sink[threadIdx.x] = s;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Every wave reads 4 KiB of a 64 KiB LDS array per iteration: four 16-byte
// reads per lane (TR false, 1 KiB per instruction, lane-contiguous) or eight
// transposing 8-byte reads (TR true, 512 B per instruction), at a rotating
// offset, folded into a value that is stored only in the fixed-pattern case.
template <bool TR>
__global__ __launch_bounds__(1024) void lds_kernel(int iters, u32x4* sink) {
  __shared__ __attribute__((aligned(16))) u32x4 s[4096];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4096; i += blockDim.x) s[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int it = 0; it < iters; ++it) {
    const int c0 = (it * 4 + wave * 5) & 63;  // first 1 KiB chunk of this iteration
    if constexpr (!TR) {
#pragma unroll
      for (int u = 0; u < 4; ++u) acc ^= s[((c0 + u) & 63) * 64 + lane];
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const char* p = reinterpret_cast<const char*>(s) + ((c0 * 2 + u) & 127) * 512 + lane * 8;
        const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
        acc.x ^= (uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16);
        acc.y ^= (uint32_t)(uint16_t)r[2] | ((uint32_t)(uint16_t)r[3] << 16);
      }
    }
  }
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0x85ebca6bu && acc.w == 0xc2b2ae35u)
    sink[threadIdx.x] = acc;
}

// Workgroup b reads region b % 8 of `region16` 16-byte vectors, `passes`
// times: workgroups run on XCD b % 8, so each XCD rereads one region, which
// its L2 holds after the first pass.  Every wave instruction moves 1 KiB:
// into registers, eight in flight per lane (TO_LDS false), or straight into
// LDS (global_load_lds_dwordx4) in groups of four into a per-wave double
// buffer, each group read back once the group after it has been issued and
// the group itself has landed.
template <bool TO_LDS>
__global__ __launch_bounds__(1024) void l2_kernel(const u32x4* __restrict__ p, int region16,
                                                  int passes, u32x4* sink) {
  __shared__ __attribute__((aligned(16))) u32x4 s[16 * 512];  // 16 waves x 8 KiB
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const u32x4* r = p + (size_t)(blockIdx.x % 8) * region16;
  u32x4* mine = s + wave * 512;
  for (int i = lane; i < 512; i += 64) mine[i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int chunks = region16 / 64;  // 1 KiB chunks
  for (int ps = 0; ps < passes; ++ps) {
    if constexpr (!TO_LDS) {
      for (int c = wave * 8; c + 7 < chunks; c += nw * 8) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = r[(c + u) * 64 + lane];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u];
      }
    } else {
      int buf = 0;
      for (int c = wave * 4; c + 3 < chunks; c += nw * 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          __builtin_amdgcn_global_load_lds(r + (c + u) * 64 + lane, mine + buf * 256 + u * 64, 16,
                                           0, 0);
        __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4): the previous group has landed
        const u32x4* prev = mine + (buf ^ 1) * 256;
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= prev[u * 64 + lane];
        buf ^= 1;
      }
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
    }
  }
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0x85ebca6bu && acc.w == 0xc2b2ae35u)
    sink[threadIdx.x] = acc;
}

}  // namespace

// LDS read rate: n_wg workgroups of `threads` threads (64..1024, a multiple of
// 64), each wave reading 4 KiB of LDS per iteration with 16-byte reads
// (transposed == 0) or transposing 8-byte reads (transposed != 0).  sink:
// device memory of at least 16 KiB, written only in the fixed-pattern case.
// Returns 0, or a hipError_t code.
extern "C" int g4probe_lds(int transposed, int n_wg, int threads, int iters, void* sink,
                           void* stream) {
  if (!sink || n_wg <= 0 || iters <= 0 || threads < 64 || threads > 1024 || threads % 64)
    return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (transposed)
    hipLaunchKernelGGL(lds_kernel<true>, dim3(n_wg), dim3(threads), 0, s, iters,
                       static_cast<u32x4*>(sink));
  else
    hipLaunchKernelGGL(lds_kernel<false>, dim3(n_wg), dim3(threads), 0, s, iters,
                       static_cast<u32x4*>(sink));
  return (int)hipGetLastError();
}

// L2 -> CU load rate: n_wg workgroups of `threads` threads (64..1024, a
// multiple of 64) reread region (workgroup % 8) of `region_bytes` (a multiple
// of 1 KiB) at device pointer p, `passes` times, into registers (to_lds == 0)
// or into LDS (to_lds != 0).  p must hold 8 regions.  sink: device memory of
// at least 16 KiB, written only in the fixed-pattern case.  Returns 0, or a
// hipError_t code.
extern "C" int g4probe_l2(int to_lds, const void* p, uint64_t region_bytes, int n_wg, int threads,
                          int passes, void* sink, void* stream) {
  if (!p || !sink || n_wg <= 0 || passes <= 0 || threads < 64 || threads > 1024 ||
      threads % 64 || region_bytes == 0 || region_bytes % 1024 || region_bytes > (1ull << 30))
    return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int region16 = (int)(region_bytes / 16);
  if (to_lds)
    hipLaunchKernelGGL(l2_kernel<true>, dim3(n_wg), dim3(threads), 0, s,
                       static_cast<const u32x4*>(p), region16, passes, static_cast<u32x4*>(sink));
  else
    hipLaunchKernelGGL(l2_kernel<false>, dim3(n_wg), dim3(threads), 0, s,
                       static_cast<const u32x4*>(p), region16, passes, static_cast<u32x4*>(sink));
  return (int)hipGetLastError();
}

// Runs n_wg workgroups of `threads` threads (256: one wave per SIMD, 512:
// two), each wave issuing `iters` rounds of `chains` (4 or 8) independent
// 16x16x32 bf16 MFMAs.  sink: device memory of at least 2 KiB, written only
// in the fixed-pattern case.  Returns 0, or a hipError_t code.
extern "C" int g4probe_mfma(int n_wg, int threads, int chains, int iters, void* sink,
                            void* stream) {
  if (!sink || n_wg <= 0 || iters <= 0 || (threads != 256 && threads != 512) ||
      (chains != 4 && chains != 8))
    return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (chains == 4)
    hipLaunchKernelGGL((mfma_kernel<4>), dim3(n_wg), dim3(threads), 0, s, iters,
                       static_cast<float*>(sink));
  else
    hipLaunchKernelGGL((mfma_kernel<8>), dim3(n_wg), dim3(threads), 0, s, iters,
                       static_cast<float*>(sink));
  return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 16) at device pointer p with n_wg workgroups of
// 256 threads, with the non-temporal hint when `nontemporal` is set.  sink:
// device memory of at least 4 KiB, written only in the fixed-pattern case.
// Returns 0, or a hipError_t code.
extern "C" int g4probe_read(const void* p, uint64_t bytes, int nontemporal, int n_wg, void* sink,
                            void* stream) {
  if (!p || !sink || bytes % 16 || n_wg <= 0) return (int)hipErrorInvalidValue;
  const size_t n = bytes / 16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nontemporal)
    hipLaunchKernelGGL((read_kernel<true, 8>), dim3(n_wg), dim3(256), 0, s,
                       static_cast<const u32x4*>(p), n, static_cast<u32x4*>(sink));
  else
    hipLaunchKernelGGL((read_kernel<false, 8>), dim3(n_wg), dim3(256), 0, s,
                       static_cast<const u32x4*>(p), n, static_cast<u32x4*>(sink));
  return (int)hipGetLastError();
}
