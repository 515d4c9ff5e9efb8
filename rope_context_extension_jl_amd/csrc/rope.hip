// Absolute RoPE applied in place: the step that writes keys into the
// absolute-position KV cache ("KV cache invariant" paragraph of the r9-hu
// digest, Method). Memory-bound: one read and one write of x.
//
// Layout: x [T, H, d] row-major. Thread (token t, pair group c) owns the
// pairs (8c .. 8c+7, d/2 + 8c .. d/2 + 8c + 7): it computes the 8 cos/sin
// once and applies them to every head of the token, so the float64 angle
// work is amortised over H heads.
#include "jl_internal.hpp"

namespace jl {

__device__ inline int find_seq(const int32_t* cu, int B, int t) {
  // largest b with cu[b] <= t (cu is non-decreasing, cu[0] = 0)
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <bool F32>
__global__ void __launch_bounds__(256) rope_apply_kernel(void* __restrict__ x, int T, int H, int d,
                                                         const int32_t* __restrict__ cu, int B,
                                                         int64_t pos_offset, RopeFreqs fr) {
  const int groups = d / 16;  // pair groups of 8 per token
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)T * groups) return;
  const int t = (int)(gid / groups);
  const int c = (int)(gid % groups);
  int64_t p = pos_offset + t;
  if (cu) p = pos_offset + (t - cu[find_seq(cu, B, t)]);
  float cs[8], sn[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) rope_cs((double)p, fr.w(8 * c + j), cs[j], sn[j]);
  const int half = d / 2;
  for (int h = 0; h < H; ++h) {
    const int64_t base = ((int64_t)t * H + h) * d;
    if constexpr (F32) {
      float* xr = (float*)x + base;
      float4 a0 = *(const float4*)(xr + 8 * c), a1 = *(const float4*)(xr + 8 * c + 4);
      float4 b0 = *(const float4*)(xr + half + 8 * c), b1 = *(const float4*)(xr + half + 8 * c + 4);
      float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      float ra[8], rb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ra[j] = a[j] * cs[j] - b[j] * sn[j];
        rb[j] = a[j] * sn[j] + b[j] * cs[j];
      }
      *(float4*)(xr + 8 * c) = make_float4(ra[0], ra[1], ra[2], ra[3]);
      *(float4*)(xr + 8 * c + 4) = make_float4(ra[4], ra[5], ra[6], ra[7]);
      *(float4*)(xr + half + 8 * c) = make_float4(rb[0], rb[1], rb[2], rb[3]);
      *(float4*)(xr + half + 8 * c + 4) = make_float4(rb[4], rb[5], rb[6], rb[7]);
    } else {
      uint16_t* xr = (uint16_t*)x + base;
      uint4 av = *(const uint4*)(xr + 8 * c);
      uint4 bv = *(const uint4*)(xr + half + 8 * c);
      const uint16_t* ap = (const uint16_t*)&av;
      const uint16_t* bp = (const uint16_t*)&bv;
      uint16_t ro[8], rq[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float a = bf16_bits_to_f32(ap[j]), b = bf16_bits_to_f32(bp[j]);
        ro[j] = f32_to_bf16_bits(a * cs[j] - b * sn[j]);
        rq[j] = f32_to_bf16_bits(a * sn[j] + b * cs[j]);
      }
      *(uint4*)(xr + 8 * c) = *(const uint4*)ro;
      *(uint4*)(xr + half + 8 * c) = *(const uint4*)rq;
    }
  }
}

hipError_t launch_rope_apply(void* x, int64_t T, int H, int d, const int32_t* cu, int B,
                             int64_t pos_offset, const RopeFreqs& fr, int is_f32,
                             hipStream_t st) {
  const int64_t threads = T * (d / 16);
  const int blocks = (int)((threads + 255) / 256);
  if (is_f32)
    hipLaunchKernelGGL(rope_apply_kernel<true>, dim3(blocks), dim3(256), 0, st, x, (int)T, H, d,
                       cu, B, pos_offset, fr);
  else
    hipLaunchKernelGGL(rope_apply_kernel<false>, dim3(blocks), dim3(256), 0, st, x, (int)T, H, d,
                       cu, B, pos_offset, fr);
  return hipGetLastError();
}

}  // namespace jl
