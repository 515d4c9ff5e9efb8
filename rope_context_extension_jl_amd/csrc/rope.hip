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
  // Heads in groups of HG: all loads of a group are issued before its first
  // store (the rows are distinct, but in place the compiler cannot know that
  // a store does not feed a later load), so each thread keeps HG rows in
  // flight instead of one.
  constexpr int HG = 4;
  for (int h0 = 0; h0 < H; h0 += HG) {
    if constexpr (F32) {
      float4 a[HG][2], b[HG][2];
#pragma unroll
      for (int u = 0; u < HG; ++u)
        if (h0 + u < H) {
          const float* xr = (const float*)x + ((int64_t)t * H + h0 + u) * d;
          a[u][0] = *(const float4*)(xr + 8 * c);
          a[u][1] = *(const float4*)(xr + 8 * c + 4);
          b[u][0] = *(const float4*)(xr + half + 8 * c);
          b[u][1] = *(const float4*)(xr + half + 8 * c + 4);
        }
#pragma unroll
      for (int u = 0; u < HG; ++u)
        if (h0 + u < H) {
          float* xr = (float*)x + ((int64_t)t * H + h0 + u) * d;
          const float av[8] = {a[u][0].x, a[u][0].y, a[u][0].z, a[u][0].w,
                               a[u][1].x, a[u][1].y, a[u][1].z, a[u][1].w};
          const float bv[8] = {b[u][0].x, b[u][0].y, b[u][0].z, b[u][0].w,
                               b[u][1].x, b[u][1].y, b[u][1].z, b[u][1].w};
          float ra[8], rb[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            ra[j] = av[j] * cs[j] - bv[j] * sn[j];
            rb[j] = av[j] * sn[j] + bv[j] * cs[j];
          }
          *(float4*)(xr + 8 * c) = make_float4(ra[0], ra[1], ra[2], ra[3]);
          *(float4*)(xr + 8 * c + 4) = make_float4(ra[4], ra[5], ra[6], ra[7]);
          *(float4*)(xr + half + 8 * c) = make_float4(rb[0], rb[1], rb[2], rb[3]);
          *(float4*)(xr + half + 8 * c + 4) = make_float4(rb[4], rb[5], rb[6], rb[7]);
        }
    } else {
      uint4 av[HG], bv[HG];
#pragma unroll
      for (int u = 0; u < HG; ++u)
        if (h0 + u < H) {
          const uint16_t* xr = (const uint16_t*)x + ((int64_t)t * H + h0 + u) * d;
          av[u] = *(const uint4*)(xr + 8 * c);
          bv[u] = *(const uint4*)(xr + half + 8 * c);
        }
#pragma unroll
      for (int u = 0; u < HG; ++u)
        if (h0 + u < H) {
          uint16_t* xr = (uint16_t*)x + ((int64_t)t * H + h0 + u) * d;
          const uint16_t* ap = (const uint16_t*)&av[u];
          const uint16_t* bp = (const uint16_t*)&bv[u];
          uint16_t ro[8], rq[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float a = bf16_bits_to_f32(ap[j]), b = bf16_bits_to_f32(bp[j]);
            ro[j] = f32_to_bf16_bits(a * cs[j] - b * sn[j]);
            rq[j] = f32_to_bf16_bits(a * sn[j] + b * cs[j]);
          }
          *(uint4*)(xr + 8 * c) = *(const uint4*)ro;
          *(uint4*)(xr + half + 8 * c) = *(const uint4*)rq;
        }
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
