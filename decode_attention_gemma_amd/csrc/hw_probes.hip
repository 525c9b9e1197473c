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

}  // namespace

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
