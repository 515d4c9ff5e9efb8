// Inclusion-exclusion merge, Eq. 7 (r9-hu digest of Jet-Long, Method,
// "Inclusion-exclusion prefill"; Sec. 3.3 Eq. 7 in the pith.science review):
//   O = (W_A O_A + W_B O_B - W_C O_C) / (W_A + W_B - W_C),
//   W_X = exp(l_X - M), M = max(l_A, l_B, l_C).
// Pass A: window keys, absolute RoPE; B: every causal key, remapped RoPE;
// C: window keys, remapped RoPE. B minus C is the remote key set.
// Numerics: the weights are formed after the max shift and the subtraction
// is done in linear space, in float64 here (the pass outputs themselves carry
// fp32 rounding); the denominator is taken as W_A + max(W_B - W_C, 0)
// (exactly W_A + W_B - W_C in real arithmetic, where W_B >= W_C). The
// per-row cancellation ratio (W_B + W_C) / denominator is stored so callers
// can see how much the subtraction amplifies the passes' rounding.
#include "jl_internal.hpp"

namespace jl {

template <bool OUT_F32>
__global__ void __launch_bounds__(256) ie_merge_kernel(const float* __restrict__ ob,
                                                       const float* __restrict__ lb,
                                                       void* __restrict__ o, float* __restrict__ lse,
                                                       float* __restrict__ ratio, int T, int Hq,
                                                       int D) {
  const int per_row = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)T * Hq * per_row) return;
  const int c = (int)(gid % per_row);
  const int64_t th = gid / per_row;  // t * Hq + h
  const int h = (int)(th % Hq);
  const int64_t t = th / Hq;
  const int64_t on = (int64_t)T * Hq * D, ln = (int64_t)T * Hq;
  const int64_t li = (int64_t)h * T + t;
  const double la = lb[li], lbb = lb[ln + li], lc = lb[2 * ln + li];
  const double M = fmax(fmax(la, lbb), lc);
  const double wa = exp(la - M), wb = exp(lbb - M), wc = exp(lc - M);
  const double den = wa + fmax(wb - wc, 0.0);
  const double inv = 1.0 / den;
  const int64_t oi = th * D + 4 * c;
  const float4 A = *(const float4*)(ob + oi);
  const float4 Bv = *(const float4*)(ob + on + oi);
  const float4 C = *(const float4*)(ob + 2 * on + oi);
  const float r[4] = {(float)((wa * A.x + wb * Bv.x - wc * C.x) * inv),
                      (float)((wa * A.y + wb * Bv.y - wc * C.y) * inv),
                      (float)((wa * A.z + wb * Bv.z - wc * C.z) * inv),
                      (float)((wa * A.w + wb * Bv.w - wc * C.w) * inv)};
  if (OUT_F32) {
    *(float4*)((float*)o + oi) = make_float4(r[0], r[1], r[2], r[3]);
  } else {
    uint16_t pk[4];
    for (int e = 0; e < 4; ++e) pk[e] = f32_to_bf16_bits(r[e]);
    *(uint2*)((uint16_t*)o + oi) = *(const uint2*)pk;
  }
  if (c == 0) {
    if (lse) lse[li] = (float)(M + log(den));
    ratio[li] = (float)((wb + wc) / den);
  }
}

hipError_t launch_ie_merge(void* o, float* lse, int out_f32, int64_t T, int Hq, int d, void* ws,
                           const PrefillLayout& lay, hipStream_t st) {
  char* w = (char*)ws;
  const int64_t n = T * Hq * (d / 4);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  const float* ob = (const float*)(w + lay.ie_o);
  const float* lb = (const float*)(w + lay.ie_lse);
  float* ratio = (float*)(w + lay.ie_ratio);
  if (out_f32)
    hipLaunchKernelGGL(ie_merge_kernel<true>, dim3(blocks), dim3(256), 0, st, ob, lb, o, lse,
                       ratio, (int)T, Hq, d);
  else
    hipLaunchKernelGGL(ie_merge_kernel<false>, dim3(blocks), dim3(256), 0, st, ob, lb, o, lse,
                       ratio, (int)T, Hq, d);
  return hipGetLastError();
}

}  // namespace jl
