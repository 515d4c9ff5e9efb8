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

// Contiguous chunks: workgroup b reads chunks b, b + grid, ... of 256 x 8
// 16-byte vectors (32 KiB); each thread issues its eight loads (each wave's
// load covers 1 KiB contiguously) before using any, so every CU keeps 8 KiB
// per wave in flight; NT adds the nontemporal hint (streamed lines are not
// kept in the caches).
template <bool NT>
__global__ void __launch_bounds__(256) calib_read_chunk_kernel(const cu32x4* __restrict__ p,
                                                               size_t n16, uint32_t* sink) {
  constexpr int U = 8;
  cu32x4 acc = {0u, 0u, 0u, 0u};
  const size_t chunk = (size_t)256 * U;
  const size_t nchunks = n16 / chunk;
  for (size_t cidx = blockIdx.x; cidx < nchunks; cidx += gridDim.x) {
    const cu32x4* q = p + cidx * chunk + threadIdx.x;
    cu32x4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = NT ? __builtin_nontemporal_load(q + 256 * k) : q[256 * k];
#pragma unroll
    for (int k = 0; k < U; ++k) acc ^= v[k];
  }
  // the tail that does not fill a chunk
  for (size_t i = nchunks * chunk + (size_t)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * 256)
    acc ^= p[i];
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[0] = 1u;
}

// Direct global -> LDS transfers (16 bytes per lane, no registers), the way
// the decode kernel streams its values: each wave keeps transferring 1 KiB
// blocks of its workgroup's chunk into its own LDS window; the transfers are
// never read back except one word at the end (so the work stays), and the
// memory counter limits how many are in flight. Chunk c (64 KiB) is read by
// workgroup c mod grid. NT: with the nontemporal hint.
template <bool NT>
__global__ void __launch_bounds__(256) calib_read_lds_kernel(const cu32x4* __restrict__ p,
                                                             size_t n16, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint8_t win[4][16 * 1024];
  constexpr int PER_WAVE = 16;  // 1 KiB transfers per wave per chunk
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const size_t chunk = (size_t)4 * PER_WAVE * 64;  // 16-byte vectors per chunk (64 KiB)
  const size_t nchunks = n16 / chunk;
  for (size_t cidx = blockIdx.x; cidx < nchunks; cidx += gridDim.x) {
    const cu32x4* q = p + cidx * chunk + (size_t)wave * PER_WAVE * 64 + lane;
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k)
      __builtin_amdgcn_global_load_lds((const void*)(q + 64 * k),
                                       (__attribute__((address_space(3))) void*)(win[wave] +
                                                                                 1024 * k),
                                       16, 0, NT ? 2 : 0);  // 2: the nontemporal hint
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t x = *(const uint32_t*)(win[wave] + 16 * lane);
  for (size_t i = nchunks * chunk + (size_t)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * 256)
    x ^= p[i].x;
  if (x == 0x9e3779b9u) sink[0] = 1u;
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
                             int variant, hipStream_t st) {
  const cu32x4* p = (const cu32x4*)src;
  const size_t n = bytes / 16;
  if (variant == 1)
    hipLaunchKernelGGL(calib_read_chunk_kernel<true>, dim3(blocks), dim3(256), 0, st, p, n, sink);
  else if (variant == 2)
    hipLaunchKernelGGL(calib_read_lds_kernel<false>, dim3(blocks), dim3(256), 0, st, p, n, sink);
  else if (variant == 3)
    hipLaunchKernelGGL(calib_read_chunk_kernel<false>, dim3(blocks), dim3(256), 0, st, p, n,
                       sink);
  else if (variant == 4)
    hipLaunchKernelGGL(calib_read_lds_kernel<true>, dim3(blocks), dim3(256), 0, st, p, n, sink);
  else
    hipLaunchKernelGGL(calib_read_kernel, dim3(blocks), dim3(256), 0, st, p, bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_calib_mfma(float* sink, int blocks, int iters, hipStream_t st) {
  hipLaunchKernelGGL(calib_mfma_kernel, dim3(blocks), dim3(256), 0, st, sink, iters);
  return hipGetLastError();
}

}  // namespace jl
