// Bifocal prefill for fp32 I/O: a plain VALU path (no matrix cores) used
// for the fp32 configuration, where results must agree with the float64
// definition to ~1e-5. Same schedule, routing and masks as the bf16 kernel
// (r9-hu digest of Jet-Long, Method, Eq. 1 and "Dynamic group size").
//
// Pre-pass: raw keys rotated once to absolute and remapped positions (fp32
// arithmetic, float64-reduced angles) into the padded head-major workspace.
// Attention: one wave per 64 query rows of one head; each lane owns a row,
// keeps both rotated query vectors and its accumulator in registers, and
// walks 32-key chunks staged in LDS with an exact-exp online softmax.
#include "jl_internal.hpp"

namespace jl {

__device__ inline int seq_of_padded_row32(const SeqInfo* seqs, int B, int r) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (seqs[mid].pad_off <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int D>
__global__ void __launch_bounds__(256) prefill_prep_f32_kernel(
    const float* __restrict__ xk, float* __restrict__ kcache, const SeqInfo* __restrict__ seqs,
    const int* __restrict__ hdr, int B, int Hkv, int R, int need_rem, int cont,
    float* __restrict__ kabs,
    float* __restrict__ krem, RopeFreqs fr) {
  constexpr int GROUPS = D / 16;            // 8 pairs per thread
  constexpr int ROWS_PER_PASS = 256 / GROUPS;
  const int r0 = blockIdx.x * 64;
  if (r0 >= hdr[2]) return;
  const SeqInfo sq = seqs[seq_of_padded_row32(seqs, B, r0)];
  for (int pass = 0; pass < 64 / ROWS_PER_PASS; ++pass) {
    const int i = pass * ROWS_PER_PASS + threadIdx.x / GROUPS;
    const int c = threadIdx.x % GROUPS;
    const int r = r0 + i;
    const int trel = r - sq.pad_off;
    const bool valid = trel < sq.len;
    float ca[8], sa[8], cr[8], sr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      rope_cs((double)trel, fr.w(8 * c + j), ca[j], sa[j]);
      if (need_rem) rope_cs(remap_pos(trel, sq.G, cont), fr.w(8 * c + j), cr[j], sr[j]);
    }
    for (int g = 0; g < Hkv; ++g) {
      float x0[8], x1[8];
      const float* src = xk + ((int64_t)(sq.start + (valid ? trel : 0)) * Hkv + g) * D;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x0[j] = valid ? src[8 * c + j] : 0.f;
        x1[j] = valid ? src[D / 2 + 8 * c + j] : 0.f;
      }
      float* da = kabs + ((int64_t)g * R + r) * D;
      float* dr = krem + ((int64_t)g * R + r) * D;
      float* dc = kcache ? kcache + ((int64_t)(sq.start + trel) * Hkv + g) * D : nullptr;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float y0 = x0[j] * ca[j] - x1[j] * sa[j], y1 = x0[j] * sa[j] + x1[j] * ca[j];
        da[8 * c + j] = y0;
        da[D / 2 + 8 * c + j] = y1;
        if (need_rem) {
          dr[8 * c + j] = x0[j] * cr[j] - x1[j] * sr[j];
          dr[D / 2 + 8 * c + j] = x0[j] * sr[j] + x1[j] * cr[j];
        }
        if (dc && valid) {
          dc[8 * c + j] = y0;
          dc[D / 2 + 8 * c + j] = y1;
        }
      }
    }
  }
}

hipError_t launch_prefill_prep_f32(const void* xk, void* kcache_out, int64_t T, int B, int Hkv,
                                   int d, int need_rem, int cont, const RopeFreqs& fr, void* ws,
                                   const PrefillLayout& lay, hipStream_t st) {
  char* w = (char*)ws;
  const int blocks = (int)(lay.R / 64);
  auto* seqs = (const SeqInfo*)(w + lay.seqs);
  auto* hdr = (const int*)(w + lay.hdr);
  if (d == 64)
    hipLaunchKernelGGL(prefill_prep_f32_kernel<64>, dim3(blocks), dim3(256), 0, st,
                       (const float*)xk, (float*)kcache_out, seqs, hdr, B, Hkv, (int)lay.R,
                       need_rem, cont, (float*)(w + lay.kabs), (float*)(w + lay.krem), fr);
  else
    hipLaunchKernelGGL(prefill_prep_f32_kernel<128>, dim3(blocks), dim3(256), 0, st,
                       (const float*)xk, (float*)kcache_out, seqs, hdr, B, Hkv, (int)lay.R,
                       need_rem, cont, (float*)(w + lay.kabs), (float*)(w + lay.krem), fr);
  (void)T;
  return hipGetLastError();
}

struct Pf32Args {
  const float* xq;
  const float* v;
  const float* kabs;
  const float* krem;
  float* o;
  float* lse;
  const SeqInfo* seqs;
  const int* hdr;
  const int* order;
  const int* tbase;
  int T, R, Hq, Hkv, w0;
  int cont;  // remote map x / G (real) instead of floor(x / G)
  float scale;
  RopeFreqs fr;
};

template <int D, int PASS>
__global__ void __launch_bounds__(64) prefill_f32_kernel(Pf32Args a) {
  constexpr int BN = PF32_BN;
  __shared__ float Ka[BN][D], Kr[BN][D], Vv[BN][D], Sc[BN][64];
  const int slot = blockIdx.x / a.Hq, head = blockIdx.x % a.Hq;
  if (slot >= a.hdr[0]) return;
  int t;
  {
    int lo = 0, hi = a.hdr[1] - 1;
    while (lo < hi) {
      int mid = (lo + hi) >> 1;
      if (a.tbase[mid] <= slot) hi = mid; else lo = mid + 1;
    }
    t = lo;
  }
  const SeqInfo sq = a.seqs[a.order[slot - a.tbase[t]]];
  const int g = head / (a.Hq / a.Hkv);
  const int lane = threadIdx.x;
  const int q0 = t * PF32_BM;
  const int q1 = min(q0 + PF32_BM, sq.len) - 1;
  const int myq = q0 + lane;
  const bool qvalid = myq < sq.len;
  constexpr bool kAbs = PASS == PASS_FUSED || PASS == PASS_PLAIN || PASS == PASS_IE_A;
  constexpr bool kRem = PASS == PASS_FUSED || PASS == PASS_IE_B || PASS == PASS_IE_C;
  constexpr bool kWindow = PASS == PASS_IE_A || PASS == PASS_IE_C;

  float qa[D], qr[D], acc[D];
  {
    const float* qp = a.xq + ((int64_t)(sq.start + (qvalid ? myq : 0)) * a.Hq + head) * D;
    const double fq = remap_pos(myq, sq.G, a.cont);
#pragma unroll
    for (int i = 0; i < D / 2; ++i) {
      const float x0 = qvalid ? qp[i] : 0.f, x1 = qvalid ? qp[i + D / 2] : 0.f;
      float c, s;
      if (kAbs) {
        rope_cs((double)myq, a.fr.w(i), c, s);
        qa[i] = x0 * c - x1 * s;
        qa[i + D / 2] = x0 * s + x1 * c;
      }
      if (kRem) {
        rope_cs(fq, a.fr.w(i), c, s);
        qr[i] = x0 * c - x1 * s;
        qr[i + D / 2] = x0 * s + x1 * c;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < D; ++i) acc[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float* kag = a.kabs + ((int64_t)g * a.R + sq.pad_off) * D;
  const float* krg = a.krem + ((int64_t)g * a.R + sq.pad_off) * D;
  const int nkc = q1 / BN + 1;
  for (int jc = 0; jc < nkc; ++jc) {
    const int k0 = jc * BN;
    const int cls = tile_class(q0, q1, k0, min(k0 + BN, sq.len) - 1, a.w0);
    if (kWindow && (cls & 3) == TC_REMOTE) continue;
    __syncthreads();
    for (int e = lane; e < BN * D; e += 64) {
      const int kr = e / D, dd = e % D;
      if (kAbs) Ka[kr][dd] = kag[(int64_t)(k0 + kr) * D + dd];
      if (kRem) Kr[kr][dd] = krg[(int64_t)(k0 + kr) * D + dd];
      const int kt = k0 + kr;
      Vv[kr][dd] = kt < sq.len ? a.v[((int64_t)(sq.start + kt) * a.Hkv + g) * D + dd] : 0.f;
    }
    __syncthreads();
    float mt = -INFINITY;
#pragma unroll 1
    for (int kr = 0; kr < BN; ++kr) {
      const int kk = k0 + kr;
      const int dist = myq - kk;
      bool use_rem;
      if (PASS == PASS_FUSED) use_rem = dist > a.w0;
      else use_rem = kRem;
      float s = 0.f;
      if (use_rem) {
#pragma unroll
        for (int i = 0; i < D; ++i) s = fmaf(qr[i], Kr[kr][i], s);
      } else {
#pragma unroll
        for (int i = 0; i < D; ++i) s = fmaf(qa[i], Ka[kr][i], s);
      }
      s *= a.scale;
      if (dist < 0 || (kWindow && dist > a.w0)) s = -INFINITY;
      Sc[kr][lane] = s;
      mt = fmaxf(mt, s);
    }
    const float m_new = fmaxf(m, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = expf(m - m_use);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < D; ++i) acc[i] *= alpha;
#pragma unroll 1
    for (int kr = 0; kr < BN; ++kr) {
      const float p = expf(Sc[kr][lane] - m_use);
      l += p;
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] = fmaf(p, Vv[kr][i], acc[i]);
    }
    m = m_new;
  }
  if (!qvalid) return;
  const int64_t row = sq.start + myq;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = a.o + (row * a.Hq + head) * D;
#pragma unroll
  for (int i = 0; i < D; ++i) op[i] = acc[i] * inv;
  if (a.lse) a.lse[(int64_t)head * a.T + row] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <int D>
static void launch_f32_pass(int pass, dim3 grid, hipStream_t st, const Pf32Args& a) {
  switch (pass) {
    case PASS_FUSED: hipLaunchKernelGGL((prefill_f32_kernel<D, PASS_FUSED>), grid, dim3(64), 0, st, a); break;
    case PASS_PLAIN: hipLaunchKernelGGL((prefill_f32_kernel<D, PASS_PLAIN>), grid, dim3(64), 0, st, a); break;
    case PASS_IE_A: hipLaunchKernelGGL((prefill_f32_kernel<D, PASS_IE_A>), grid, dim3(64), 0, st, a); break;
    case PASS_IE_B: hipLaunchKernelGGL((prefill_f32_kernel<D, PASS_IE_B>), grid, dim3(64), 0, st, a); break;
    default: hipLaunchKernelGGL((prefill_f32_kernel<D, PASS_IE_C>), grid, dim3(64), 0, st, a); break;
  }
}

hipError_t launch_prefill_f32(int pass, const void* xq, const void* v, void* o, float* lse,
                              int64_t T, int B, int Hq, int Hkv, int d, int64_t w0, float scale,
                              int cont, const RopeFreqs& fr, void* ws, const PrefillLayout& lay,
                              hipStream_t st) {
  char* w = (char*)ws;
  Pf32Args a;
  a.xq = (const float*)xq;
  a.v = (const float*)v;
  a.kabs = (const float*)(w + lay.kabs);
  a.krem = (const float*)(w + lay.krem);
  a.o = (float*)o;
  a.lse = lse;
  a.seqs = (const SeqInfo*)(w + lay.seqs);
  a.hdr = (const int*)(w + lay.hdr);
  a.order = (const int*)(w + lay.tiles);
  a.tbase = a.order + B + (lay.max_tiles + 1);
  a.T = (int)T;
  a.R = (int)lay.R;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.w0 = (int)w0;
  a.scale = scale;
  a.cont = cont;
  a.fr = fr;
  const dim3 grid((unsigned)(lay.max_tiles * Hq));
  if (d == 64) launch_f32_pass<64>(pass, grid, st, a);
  else launch_f32_pass<128>(pass, grid, st, a);
  return hipGetLastError();
}

}  // namespace jl
