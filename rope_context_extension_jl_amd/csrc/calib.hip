// Calibration kernels for the rooflines the benchmark reports next to the
// vendor peaks (not part of the attention method): the HBM read rate a plain
// streaming kernel reaches, and the bf16 matrix-core rate at the clock the
// chip sustains under a pure MFMA load.
#include "jl_internal.hpp"

namespace jl {

typedef uint32_t cu32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 cb8v __attribute__((ext_vector_type(8)));
typedef float cf32x16 __attribute__((ext_vector_type(16)));

// Grid-stride 16-byte reads, four in flight per thread, xor-reduced; the
// result reaches *sink only when it equals a value no input here produces,
// so the reads cannot be removed and nothing is written in practice.
__global__ void __launch_bounds__(256) calib_read_kernel(const cu32x4* __restrict__ p, size_t n16,
                                                         uint32_t* sink) {
  cu32x4 acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const cu32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= p[i];
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[0] = 1u;
}

// Four independent 32x32x16 bf16 MFMA chains per wave, `iters` rounds.
__global__ void __launch_bounds__(256) calib_mfma_kernel(float* sink, int iters) {
  cb8v a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.f + 0.001f * (threadIdx.x & 7) + 0.01f * i);
    b[i] = (__bf16)(0.5f - 0.01f * i);
  }
  cf32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

hipError_t launch_calib_read(const void* src, size_t bytes, uint32_t* sink, int blocks,
                             hipStream_t st) {
  hipLaunchKernelGGL(calib_read_kernel, dim3(blocks), dim3(256), 0, st, (const cu32x4*)src,
                     bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_calib_mfma(float* sink, int blocks, int iters, hipStream_t st) {
  hipLaunchKernelGGL(calib_mfma_kernel, dim3(blocks), dim3(256), 0, st, sink, iters);
  return hipGetLastError();
}

}  // namespace jl
