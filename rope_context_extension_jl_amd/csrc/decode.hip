// Single-token bifocal decode against the absolute KV cache (r9-hu digest
// of Jet-Long, Method: Eq. 1 and the "KV cache invariant" paragraph; Sec. 3.2
// Eqs. 5-6 in the pith.science review).
//
// The cache holds keys rotated at their absolute positions and is never
// written. At step pos (L = pos + 1, G from Eq. 2) a key k with pos - k > w0
// is corrected on the fly by the rotation R_{f(k) - k}, which by
// R_a R_b = R_{a+b} turns RoPE(x_k, k) into RoPE(x_k, f(k)); it is scored
// against the query rotated at f(pos). Keys inside the window are scored
// against the query rotated at pos.
//
// Split-K: workgroup (split s, KV head g) streams keys [s*n, (s+1)*n) of
// head g once, for all Hq/Hkv query heads of the group, and leaves a partial
// (max, sum, unnormalised accumulator) per query head; a second kernel merges
// the splits with LSE weights. HBM traffic is the K and V rows of keys
// 0..pos read once.
//
// Lane layout: D/8 lanes per key; lane dl holds the pairs
// (4dl .. 4dl+3, D/2 + 4dl .. D/2 + 4dl + 3), so the correction rotation is
// in-lane and a key's dot product is a D/8-lane reduction.
#include "jl_internal.hpp"

namespace jl {

struct DecArgs {
  const void* xq;  // raw query [Hq, D]
  const void* kc;  // [C, Hkv, D] absolute-rotated keys
  const void* vc;  // [C, Hkv, D]
  float* part;     // [Hq, S, D + 2]: m (log2 domain), l, acc[D]
  void* o;
  float* lse;
  int pos, Hq, Hkv, w0, G, plain, S, kps;
  float scale_log2;
  RopeFreqs fr;
};

template <bool F32>
__device__ inline void load4(const void* base, int64_t idx, float* out) {
  if constexpr (F32) {
    float4 v = *(const float4*)((const float*)base + idx);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  } else {
    uint2 v = *(const uint2*)((const uint16_t*)base + idx);
    out[0] = __uint_as_float(v.x << 16);
    out[1] = __uint_as_float(v.x & 0xffff0000u);
    out[2] = __uint_as_float(v.y << 16);
    out[3] = __uint_as_float(v.y & 0xffff0000u);
  }
}

template <bool F32>
__device__ inline float load1(const void* base, int64_t idx) {
  if constexpr (F32) return ((const float*)base)[idx];
  else return bf16_bits_to_f32(((const uint16_t*)base)[idx]);
}

template <bool F32, int D, int R>
__global__ void __launch_bounds__(256) decode_split_kernel(DecArgs a) {
  constexpr int NL = D / 8;     // lanes per key
  constexpr int KPW = 64 / NL;  // keys per wave step
  constexpr int HALF = D / 2;
  __shared__ float qa_s[R][D], qr_s[R][D];
  __shared__ float red_m[4][R], red_l[4][R];
  __shared__ float red_acc[4][R][D];
  const int s = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int dl = lane % NL, kl = lane / NL;
  const int h0 = g * R;
  const int fpos = a.pos / a.G;
  // rotated queries for the R heads of this KV group
  for (int idx = tid; idx < R * HALF; idx += 256) {
    const int hl = idx / HALF, i = idx % HALF;
    const float x0 = load1<F32>(a.xq, (int64_t)(h0 + hl) * D + i);
    const float x1 = load1<F32>(a.xq, (int64_t)(h0 + hl) * D + HALF + i);
    float c, sn;
    rope_cs((double)a.pos, a.fr.w(i), c, sn);
    qa_s[hl][i] = x0 * c - x1 * sn;
    qa_s[hl][HALF + i] = x0 * sn + x1 * c;
    rope_cs((double)fpos, a.fr.w(i), c, sn);
    qr_s[hl][i] = x0 * c - x1 * sn;
    qr_s[hl][HALF + i] = x0 * sn + x1 * c;
  }
  __syncthreads();
  float qa0[R][4], qa1[R][4], qr0[R][4], qr1[R][4];
#pragma unroll
  for (int h = 0; h < R; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qa0[h][e] = qa_s[h][4 * dl + e];
      qa1[h][e] = qa_s[h][HALF + 4 * dl + e];
      qr0[h][e] = qr_s[h][4 * dl + e];
      qr1[h][e] = qr_s[h][HALF + 4 * dl + e];
    }
  float m[R], l[R], acc0[R][4], acc1[R][4];
#pragma unroll
  for (int h = 0; h < R; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc0[h][e] = acc1[h][e] = 0.f;
  }
  double wl[4];  // this lane's four rotary frequencies (in turns for 16-bit I/O)
#pragma unroll
  for (int e = 0; e < 4; ++e) wl[e] = F32 ? a.fr.w(4 * dl + e) : a.fr.w(4 * dl + e) * kInvTwoPi;
  const int k_lo = s * a.kps;
  const int k_hi = min(k_lo + a.kps, a.pos + 1);
  for (int kb = k_lo + wave * KPW; kb < k_hi; kb += 4 * KPW) {
    const int kk = kb + kl;
    const bool valid = kk < k_hi;
    float k0[4] = {0, 0, 0, 0}, k1[4] = {0, 0, 0, 0}, v0[4] = {0, 0, 0, 0}, v1[4] = {0, 0, 0, 0};
    if (valid) {
      const int64_t row = ((int64_t)kk * a.Hkv + g) * D;
      load4<F32>(a.kc, row + 4 * dl, k0);
      load4<F32>(a.kc, row + HALF + 4 * dl, k1);
      load4<F32>(a.vc, row + 4 * dl, v0);
      load4<F32>(a.vc, row + HALF + 4 * dl, v1);
    }
    const bool remote = !a.plain && (a.pos - kk > a.w0);
    if (remote && a.G > 1) {
      const int delta = kk / a.G - kk;  // f(k) - k
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float c, sn;
        if constexpr (F32) rope_cs((double)delta, wl[e], c, sn);
        else rope_cs_turns((double)delta, wl[e], c, sn);
        const float x0 = k0[e], x1 = k1[e];
        k0[e] = x0 * c - x1 * sn;
        k1[e] = x0 * sn + x1 * c;
      }
    }
#pragma unroll
    for (int h = 0; h < R; ++h) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d = fmaf(remote ? qr0[h][e] : qa0[h][e], k0[e], d);
        d = fmaf(remote ? qr1[h][e] : qa1[h][e], k1[e], d);
      }
#pragma unroll
      for (int off = 1; off < NL; off <<= 1) d += __shfl_xor(d, off);
      const float x = valid ? d * a.scale_log2 : -INFINITY;
      const float mn = fmaxf(m[h], x);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float al = __builtin_amdgcn_exp2f(m[h] - mu);
      const float p = __builtin_amdgcn_exp2f(x - mu);
      l[h] = l[h] * al + p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc0[h][e] = acc0[h][e] * al + p * v0[e];
        acc1[h][e] = acc1[h][e] * al + p * v1[e];
      }
      m[h] = mn;
    }
  }
  // combine the KPW key sub-streams of the wave (lanes dl + NL * kl)
#pragma unroll
  for (int h = 0; h < R; ++h) {
    float mm = m[h];
#pragma unroll
    for (int off = NL; off < 64; off <<= 1) mm = fmaxf(mm, __shfl_xor(mm, off));
    const float sc = m[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[h] - mm);
    float lh = l[h] * sc;
#pragma unroll
    for (int off = NL; off < 64; off <<= 1) lh += __shfl_xor(lh, off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x0 = acc0[h][e] * sc, x1 = acc1[h][e] * sc;
#pragma unroll
      for (int off = NL; off < 64; off <<= 1) {
        x0 += __shfl_xor(x0, off);
        x1 += __shfl_xor(x1, off);
      }
      if (kl == 0) {
        red_acc[wave][h][4 * dl + e] = x0;
        red_acc[wave][h][HALF + 4 * dl + e] = x1;
      }
    }
    if (lane == 0) {
      red_m[wave][h] = mm;
      red_l[wave][h] = lh;
    }
  }
  __syncthreads();
  // combine the 4 waves and write the split's partial
  for (int idx = tid; idx < R * D; idx += 256) {
    const int h = idx / D, dd = idx % D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, red_m[w][h]);
    float lt = 0.f, at = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = red_m[w][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(red_m[w][h] - mm);
      lt += red_l[w][h] * sc;
      at += red_acc[w][h][dd] * sc;
    }
    float* pp = a.part + ((int64_t)(h0 + h) * a.S + s) * (D + 2);
    pp[2 + dd] = at;
    if (dd == 0) {
      pp[0] = mm;
      pp[1] = lt;
    }
  }
}

template <bool F32, int D>
__global__ void __launch_bounds__(D) decode_merge_kernel(DecArgs a) {
  const int h = blockIdx.x, dd = threadIdx.x;
  const float* pp = a.part + (int64_t)h * a.S * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < a.S; ++s) M = fmaxf(M, pp[(int64_t)s * (D + 2)]);
  float L = 0.f, A = 0.f;
  for (int s = 0; s < a.S; ++s) {
    const float ms = pp[(int64_t)s * (D + 2)];
    const float w = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    L += pp[(int64_t)s * (D + 2) + 1] * w;
    A += pp[(int64_t)s * (D + 2) + 2 + dd] * w;
  }
  const float out = A / L;
  if constexpr (F32) ((float*)a.o)[(int64_t)h * D + dd] = out;
  else ((uint16_t*)a.o)[(int64_t)h * D + dd] = f32_to_bf16_bits(out);
  if (a.lse && dd == 0) a.lse[h] = (M + __log2f(L)) * 0.69314718055994530942f;
}

template <bool F32, int D>
static void launch_decode_t(int R, dim3 grid, hipStream_t st, const DecArgs& a) {
  switch (R) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<F32, D, 1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<F32, D, 2>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<F32, D, 4>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((decode_split_kernel<F32, D, 8>), grid, dim3(256), 0, st, a); break;
  }
  hipLaunchKernelGGL((decode_merge_kernel<F32, D>), dim3(a.Hq), dim3(D), 0, st, a);
}

hipError_t launch_decode(const void* xq, const void* kc, const void* vc, void* o, float* lse,
                         int64_t pos, int Hq, int Hkv, int d, int64_t w0, int64_t G, float scale,
                         const RopeFreqs& fr, int plain, int is_f32, int num_splits, void* ws,
                         hipStream_t st) {
  DecArgs a;
  a.xq = xq;
  a.kc = kc;
  a.vc = vc;
  a.part = (float*)ws;
  a.o = o;
  a.lse = lse;
  a.pos = (int)pos;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.w0 = (int)w0;
  a.G = (int)G;
  a.plain = plain;
  const int keys = (int)pos + 1;
  int kps = (keys + num_splits - 1) / num_splits;
  a.S = (keys + kps - 1) / kps;  // no empty split
  a.kps = kps;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.fr = fr;
  const int R = Hq / Hkv;
  const dim3 grid(a.S, Hkv);
  if (is_f32) {
    if (d == 64) launch_decode_t<true, 64>(R, grid, st, a);
    else launch_decode_t<true, 128>(R, grid, st, a);
  } else {
    if (d == 64) launch_decode_t<false, 64>(R, grid, st, a);
    else launch_decode_t<false, 128>(R, grid, st, a);
  }
  return hipGetLastError();
}

}  // namespace jl
