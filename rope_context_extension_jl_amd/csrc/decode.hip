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
// Split-K: the keys 0..pos of every KV head are cut into ranges, each
// streamed once for all Hq/Hkv query heads of the group, leaving a partial
// (max, sum, unnormalised accumulator) per query head; the partials are
// merged with LSE weights. HBM traffic is the K and V rows of keys 0..pos
// read once. bf16: one workgroup per (KV head, range) and the merge folded
// into the same kernel (the last range of a head to finish merges). float32:
// one workgroup per (split, KV head) and a second merge kernel.
#include "jl_internal.hpp"

namespace jl {

struct DecArgs {
  const void* xq;  // raw query [Hq, D]
  const void* kc;  // [C, Hkv, D] absolute-rotated keys
  const void* vc;  // [C, Hkv, D]
  float* part;     // float32: [Hq, S, D + 2]: m (log2 domain), l, acc[D]
  float* rec;      // bf16: range records (see dec_recf); same memory as part
  int* tickets;    // bf16: arrival count per (sequence, KV head), zero between calls
  void* o;
  float* lse;
  int pos, Hq, Hkv, w0, G, plain, S, kps;
  int cont;        // remote map x / G (real) instead of floor(x / G)
  double fk_rel;   // with cont: f(k) - k = k * fk_rel, fk_rel = 1 / G - 1
  float scale_log2;
  RopeFreqs fr;
  // batched decode: per-sequence position and first cache row (device), the
  // bound on pos + 1 the split plan was made for, the cache's row count and
  // w_pre (each sequence takes G from its own L = pos + 1)
  const int* bpos;
  const int* bstart;
  int max_keys;
  int64_t cap_rows;
  int64_t w_pre;
};

// One sequence's view of the arguments: a single decode takes it from the
// scalars; a batched one from the per-sequence arrays, b being the grid's
// batch index. ok is false for a batch entry whose position or cache rows
// fall outside the bounds the caller gave: the kernels skip it and the merge
// writes NaN for it, so no read goes out of bounds.
struct DecSeq {
  int pos, G;
  double fk_rel;
  bool ok;
  const char* xq;  // this sequence's query rows [Hq, D]
  const char* kc;  // its cache row 0 [.., Hkv, D]
  const char* vc;
  float* part;     // its partials [Hq, S, D + 2]
};

template <bool BATCH>
__device__ __forceinline__ DecSeq dec_seq(const DecArgs& a, int b, int D, int esz) {
  DecSeq q;
  int64_t row0 = 0;
  if constexpr (BATCH) {
    const int p = a.bpos[b], st = a.bstart[b];
    q.ok = p >= 0 && p < a.max_keys && st >= 0 && (int64_t)st + p < a.cap_rows;
    q.pos = q.ok ? p : 0;
    q.G = (int)(((int64_t)q.pos + a.w_pre) / a.w_pre);  // Eq. 2 with L = pos + 1
    q.fk_rel = 1.0 / (double)q.G - 1.0;
    row0 = q.ok ? st : 0;
  } else {
    q.pos = a.pos;
    q.G = a.G;
    q.fk_rel = a.fk_rel;
    q.ok = true;
  }
  q.xq = (const char*)a.xq + (int64_t)b * a.Hq * D * esz;
  q.kc = (const char*)a.kc + row0 * a.Hkv * D * esz;
  q.vc = (const char*)a.vc + row0 * a.Hkv * D * esz;
  q.part = a.part + (int64_t)b * a.Hq * a.S * (D + 2);
  return q;
}

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

template <bool F32, int D, int R, bool BATCH>
__global__ void __launch_bounds__(256) decode_split_kernel(DecArgs a) {
  constexpr int NL = D / 8;     // lanes per key
  constexpr int KPW = 64 / NL;  // keys per wave step
  constexpr int HALF = D / 2;
  __shared__ float qa_s[R][D], qr_s[R][D];
  __shared__ float red_m[4][R], red_l[4][R];
  __shared__ float red_acc[4][R][D];
  const int s = blockIdx.x, g = blockIdx.y;
  const DecSeq sq = dec_seq<BATCH>(a, blockIdx.z, D, F32 ? 4 : 2);
  // workgroup-uniform exits, before any barrier
  if (!sq.ok || s * a.kps > sq.pos) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int dl = lane % NL, kl = lane / NL;
  const int h0 = g * R;
  const double fpos = remap_pos(sq.pos, sq.G, a.cont);
  // rotated queries for the R heads of this KV group
  for (int idx = tid; idx < R * HALF; idx += 256) {
    const int hl = idx / HALF, i = idx % HALF;
    const float x0 = load1<F32>(sq.xq, (int64_t)(h0 + hl) * D + i);
    const float x1 = load1<F32>(sq.xq, (int64_t)(h0 + hl) * D + HALF + i);
    float c, sn;
    rope_cs((double)sq.pos, a.fr.w(i), c, sn);
    qa_s[hl][i] = x0 * c - x1 * sn;
    qa_s[hl][HALF + i] = x0 * sn + x1 * c;
    rope_cs(fpos, a.fr.w(i), c, sn);
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
  const int k_hi = min(k_lo + a.kps, sq.pos + 1);
  for (int kb = k_lo + wave * KPW; kb < k_hi; kb += 4 * KPW) {
    const int kk = kb + kl;
    const bool valid = kk < k_hi;
    float k0[4] = {0, 0, 0, 0}, k1[4] = {0, 0, 0, 0}, v0[4] = {0, 0, 0, 0}, v1[4] = {0, 0, 0, 0};
    if (valid) {
      const int64_t row = ((int64_t)kk * a.Hkv + g) * D;
      load4<F32>(sq.kc, row + 4 * dl, k0);
      load4<F32>(sq.kc, row + HALF + 4 * dl, k1);
      load4<F32>(sq.vc, row + 4 * dl, v0);
      load4<F32>(sq.vc, row + HALF + 4 * dl, v1);
    }
    const bool remote = !a.plain && (sq.pos - kk > a.w0);
    if (remote && sq.G > 1) {
      // f(k) - k
      const double delta = a.cont ? (double)kk * sq.fk_rel : (double)(kk / sq.G - kk);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float c, sn;
        if constexpr (F32) rope_cs(delta, wl[e], c, sn);
        else rope_cs_turns(delta, wl[e], c, sn);
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
    float* pp = sq.part + ((int64_t)(h0 + h) * a.S + s) * (D + 2);
    pp[2 + dd] = at;
    if (dd == 0) {
      pp[0] = mm;
      pp[1] = lt;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 path: both products on the matrix cores, the split merge folded in.
//
// Workgroup = one KV head x one key range [s kps, (s + 1) kps) of one
// sequence, DEC_NW waves; wave w takes the range's 32-key chunks w, w + NW,
// ..., so the waves running together read neighbouring key rows. Per chunk a
// wave loads K (the A operand of S^T = K Q^T, fp16, 16x16x32 MFMAs: lane =
// one key, 8 consecutive dims) and sends V straight to a wave-private LDS
// stage. The S^T tile gives each lane one query (lane % 16) and four keys
// per 16-key block, which is the A operand of O = P V for two consecutive
// blocks; the V operand (8 keys at one dim per lane) comes from LDS with the
// transpose read ds_read_b64_tr_b16: within 16 lanes, lane i receives element
// i % 4 of the 8-byte rows addressed by lanes i / 4 + 4t, t = 0..3, so lanes
// pointing at V[key_t][4c .. 4c + 3] deliver V[key_t][own dim] for 4 keys.
// Query heads are padded to the 16 MFMA columns with zeros.
//
// At the end the waves' softmax states are merged in LDS into one record per
// (range, query head): m (log2 domain), l and the unnormalised O. The record
// is released at device scope and the workgroup takes a ticket of its
// (sequence, KV head); the last range to arrive merges all the records with
// LSE weights, writes O and the LSE and puts the ticket back to zero, so no
// second launch is needed.
//
// Remote keys (pos - k > w0) are corrected by R_{f(k) - k} (R_a R_b =
// R_{a+b} turns the absolute key RoPE(x_k, k) into RoPE(x_k, f(k))):
//   DEC_FACT (G divides 32, or the continuous map): with k = k0 + i, k0 the
//     chunk's first key (a multiple of 32), f(k) - k = (f(k0) - k0) +
//     (f(i) - i). The chunk-uniform factor moves to the query,
//     q . (R_a R_b k) = (R_{-a} q) . (R_b k): once per chunk the wave rotates
//     the raw query to f(pos) - (f(k0) - k0), one angle per frequency, shared
//     through LDS; the in-chunk factor depends on i alone and is a per-lane
//     constant.
//   DEC_GEN (any G; used for the floor map with G not dividing 32, and by
//     the batch kernel): each lane evaluates its key's angles for the
//     chunk's first 16-key block; the second block follows by one rotation
//     R_{c16}, c16 = f(k + 16) - f(k) - 16, one of two values per G picked
//     by k mod G (one value for the continuous map).
//   DEC_PLAIN (plain mode, or G = 1 where f(x) = x): no correction.
//
// Softmax: the query operand carries scale * log2(e) and the score
// accumulator starts at -m, m a per-wave reference that moves only when a
// lane's sum of bf16-rounded p over the chunk exceeds 2^8 (or on the first
// scores), so the common chunk needs no row max and no cross-lane exchange.
// A raw score that is not finite (an fp16 operand out of range) makes the
// KV head's outputs NaN.
// ---------------------------------------------------------------------------
constexpr int DEC_CHUNK = 32;  // keys per chunk
constexpr int DEC_NW = 4;      // waves per bf16 workgroup (one KV head, one key range)
constexpr int DEC_RP = 8;      // (m, l) slots at the head of a bf16 record
// Correction paths of the bf16 kernels (see below).
enum DecPath : int { DEC_PLAIN = 0, DEC_FACT = 1, DEC_GEN = 2 };

typedef _Float16 dh8v __attribute__((ext_vector_type(8)));
typedef _Float16 dh2v __attribute__((ext_vector_type(2)));
typedef __bf16 db8v __attribute__((ext_vector_type(8)));
typedef __bf16 db2v __attribute__((ext_vector_type(2)));
typedef short ds4v __attribute__((ext_vector_type(4)));
typedef float df32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t du32x4 __attribute__((ext_vector_type(4)));

constexpr float kDecSumMax = 256.f;

template <int D>
struct DecGeom {
  static constexpr int NDS = D / 32;                    // 32-dim steps of the QK product
  static constexpr int NDB = D / 16;                    // 16-dim output blocks of the PV product
  static constexpr int NC = D / 8;                      // 16-byte chunks per key row
  static constexpr int VROW = 2 * D;                    // LDS bytes per key row
  static constexpr int VLD = DEC_CHUNK * 2 * D / 1024;  // 1 KiB V transfers per chunk
  static constexpr int RPL = 64 / NC;                   // key rows per transfer
  static constexpr int VBYTES = DEC_CHUNK * VROW;       // one LDS stage
};

// LDS position of 16-byte chunk ch of key row r in a V stage: rows are
// packed (the direct-to-LDS transfers write 1 KiB contiguously) and the chunk
// index is XOR-swizzled by the row so that the transpose reads of the PV
// operand (4 rows x 32 bytes per 16 lanes) hit distinct banks.
template <int D>
__device__ __forceinline__ int dec_vswz(int r) {
  return (2 * r) & (DecGeom<D>::NC - 1);
}

// Workgroup memory of the bf16 kernels (under 80 KiB at D = 128, so two
// workgroups share a CU), as separate LDS arrays: the compiler then sees
// that the reads of one V stage, of the tables or of the query cannot alias
// the direct transfers in flight into the other stage, and does not wait for
// those. The prologue's operand tables live in the second V stages (vB),
// which no transfer touches before the key loop.
template <int D>
struct DecLds {
  uint8_t* vA;   // [DEC_NW][VBYTES] first V stage of each wave; merge scratch after the loop
  uint8_t* vB;   // [DEC_NW][VBYTES] second V stage of each wave
  float* qraw;   // [8][D] raw query rows of the group x scale log2 e (rows >= R zero)
  float2* cs;    // [DEC_NW][D / 2] DEC_FACT: the chunk's query rotation per wave;
                 // DEC_GEN: the two R_{c16} tables as fp16
  double* w2pi;  // [D / 2] omega_i / (2 pi)
  int* flag;     // [2]: a range's non-finite flag, the last-arrival flag
};

template <int D>
__device__ __forceinline__ DecLds<D> dec_lds() {
  __shared__ __attribute__((aligned(16))) uint8_t vA[DEC_NW * DecGeom<D>::VBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vB[DEC_NW * DecGeom<D>::VBYTES];
  __shared__ __attribute__((aligned(16))) float qraw[8 * D];
  __shared__ __attribute__((aligned(16))) float2 cs[DEC_NW * D / 2];
  __shared__ double w2pi[D / 2];
  __shared__ int flag[2];
  return DecLds<D>{vA, vB, qraw, cs, w2pi, flag};
}

// Per-wave constants of the key loop (all wave-uniform except the lane ids).
struct DecCtx {
  const uint16_t* kbase;  // this lane's K slice: head, dims 8 * g16 ..
  const uint16_t* vbase;  // the head's V row 0
  int64_t rstride;        // elements between consecutive keys
  int pos, w0, G, k_hi;
  int plain;      // every key local: plain mode, or G = 1 (f(x) = x)
  int cont;       // remote map x / G (real) instead of floor(x / G)
  double fk_rel;  // with cont: f(k) - k = k * fk_rel
  double fpos;    // f(pos)
  int lane, g16, r16;
};

// One chunk's K fragments (key k0 + 16 kb + r16, dims 32 ds + 8 g16 .. + 8);
// its V rows go straight to an LDS stage.
template <int D>
struct DecBuf {
  du32x4 k[2][D / 32];
};

template <int D>
struct DecState {
  df32x4 acc[D / 16];  // O: lane holds dims 16 db + r16 of queries 4 g16 + r
  df32x4 negm;         // -m in every element: the QK accumulator's start value
  float m, lsum;       // reference (log2 domain) of query r16, partial row sum
};

template <int D>
__device__ __forceinline__ void dec_qk(const dh8v (&kf)[D / 32], const dh8v (&q)[D / 32],
                                       const df32x4& c, df32x4& out) {
  out = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[0], q[0], c, 0, 0, 0);
#pragma unroll
  for (int ds = 1; ds < D / 32; ++ds)
    out = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[ds], q[ds], out, 0, 0, 0);
}

// bf16 pairs of a 16-byte vector -> 8 fp16 (exact for normal bf16 values in
// fp16 range).
__device__ __forceinline__ dh8v dec_to_f16(const du32x4& v) {
  dh8v r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (_Float16)bf16_lane(v, j);
  return r;
}

template <int D>
__device__ __forceinline__ void dec_issue_k(const DecCtx& c, int k0, DecBuf<D>& b) {
  using G = DecGeom<D>;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    // keys past the range end load the last key (finite data, masked later)
    const int key = min(k0 + 16 * kb + c.r16, c.k_hi - 1);
#pragma unroll
    for (int ds = 0; ds < G::NDS; ++ds)
      b.k[kb][ds] = __builtin_nontemporal_load((const du32x4*)(c.kbase + key * c.rstride + 32 * ds));
  }
}

// V rows of the chunk, global -> LDS stage without registers: transfer i
// writes rows RPL i .. RPL i + RPL - 1; lane L fills slot L, i.e. row
// RPL i + L / NC, swizzled chunk L % NC, so it fetches the row's chunk
// (L % NC) ^ swz(row).
template <int D>
__device__ __forceinline__ void dec_issue_v(const DecCtx& c, int k0, uint8_t* stage) {
  using G = DecGeom<D>;
#pragma unroll
  for (int i = 0; i < G::VLD; ++i) {
    const int row = G::RPL * i + c.lane / G::NC;
    const int ch = (c.lane % G::NC) ^ dec_vswz<D>(row);
    const int key = min(k0 + row, c.k_hi - 1);
    __builtin_amdgcn_global_load_lds(
        (const void*)(c.vbase + key * c.rstride + 8 * ch),
        (__attribute__((address_space(3))) void*)(stage + 1024 * i), 16, 0, 2);  // 2: nontemporal
  }
}

// p = exp2(s') of the chunk's two 16-key blocks, packed as the A operand of
// O = P V; returns the lane's sum of the rounded p.
__device__ __forceinline__ float dec_exp(const df32x4 (&st)[2], db8v& pb) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) pb[4 * kb + r] = (__bf16)__builtin_amdgcn_exp2f(st[kb][r]);
  const db2v one = {(__bf16)1.f, (__bf16)1.f};
  float ps0 =
      __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 0, 1), one, 0.f, false);
  float ps1 =
      __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 2, 3), one, 0.f, false);
  ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 4, 5), one, ps0, false);
  ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 6, 7), one, ps1, false);
  return ps0 + ps1;
}

// Wait for this wave's LDS reads and writes only (lgkmcnt 0; the vector
// memory and export counters at their maxima, so loads in flight stay).
__device__ __forceinline__ void dec_wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// One chunk: correction setup, S^T = K Q^T per 16-key block (seeded with -m),
// the lazy-reference softmax and O += P V. chk accumulates the raw scores
// (a non-finite sum flags an operand out of the fp16 range).
template <int D, int PATH>
__device__ __forceinline__ void dec_chunk(const DecCtx& c, int k0, const DecBuf<D>& b,
                                          const dh8v (&qa)[D / 32], dh8v (&qr)[D / 32],
                                          const dh2v (&tcr)[2][D / 64][4],
                                          const dh2v (&tsr)[2][D / 64][4], const DecLds<D>& sh,
                                          int wave, const uint8_t* vb, DecState<D>& st,
                                          float& chk) {
  using G = DecGeom<D>;
  constexpr int NDS = G::NDS, NDB = G::NDB, VROW = G::VROW, HALF = D / 2;
  // ---- correction setup. It depends on key indices only, so it runs before
  // the chunk's data is first touched, while its loads (and the next
  // chunk's) are in flight.
  const bool chunk_rem = PATH != DEC_PLAIN && !c.plain && c.pos - k0 > c.w0;  // block 0 has remote keys
  dh2v rc[2][NDS / 2][4], rs[2][NDS / 2][4];
  if (PATH == DEC_FACT && chunk_rem) {
    // query operand for this chunk: raw query at f(pos) - (f(k0) - k0)
    if (c.lane < HALF) {
      const double P = c.cont ? c.fpos - (double)k0 * c.fk_rel
                              : (double)(c.pos / c.G - k0 / c.G + k0);
      float cc, ss;
      rope_cs_turns(P, sh.w2pi[c.lane], cc, ss);
      sh.cs[wave * HALF + c.lane] = make_float2(cc, ss);
    }
    dec_wait_lds();
    __builtin_amdgcn_wave_barrier();
    const bool qv = c.r16 < 8;
    const float* qrow = sh.qraw + (c.r16 & 7) * D;
#pragma unroll
    for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int f = 32 * ds + 8 * c.g16 + j;
        const float2 t = sh.cs[wave * HALF + f];
        const float x0 = qv ? qrow[f] : 0.f, x1 = qv ? qrow[f + HALF] : 0.f;
        qr[ds][j] = (_Float16)(x0 * t.x - x1 * t.y);
        qr[ds + NDS / 2][j] = (_Float16)(x0 * t.y + x1 * t.x);
      }
  }
  if (PATH == DEC_GEN && chunk_rem) {
    // block 0: this lane's key, frequencies 32 ds + 8 g16 + 2 m (+ 1), as
    // fp16 pairs of neighbouring frequencies (the key fragment's layout)
    const int key = k0 + c.r16;
    const double delta = c.cont ? (double)key * c.fk_rel : (double)(key / c.G - key);
#pragma unroll
    for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float c0, s0, c1, s1;
        rope_cs_turns(delta, sh.w2pi[32 * ds + 8 * c.g16 + 2 * m], c0, s0);
        rope_cs_turns(delta, sh.w2pi[32 * ds + 8 * c.g16 + 2 * m + 1], c1, s1);
        rc[0][ds][m] = dh2v{(_Float16)c0, (_Float16)c1};
        rs[0][ds][m] = dh2v{(_Float16)s0, (_Float16)s1};
      }
    if (c.pos - (k0 + 16) > c.w0) {
      // block 1 (key + 16; block 0 is then all remote): R_{d + c16} =
      // R_d R_{c16}, c16 = f(key + 16) - f(key) - 16 takes the larger of its
      // two values when the key's residue carries (continuous map: one value)
      const int t = !c.cont && (key % c.G) + (16 % c.G) >= c.G ? 1 : 0;
      const _Float16* tt = (const _Float16*)sh.cs + 2 * t * HALF;
#pragma unroll
      for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int f = 32 * ds + 8 * c.g16 + 2 * m;
          const dh2v cst = *(const dh2v*)(tt + f), sst = *(const dh2v*)(tt + HALF + f);
          rc[1][ds][m] = rc[0][ds][m] * cst - rs[0][ds][m] * sst;
          rs[1][ds][m] = rs[0][ds][m] * cst + rc[0][ds][m] * sst;
        }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // ---- S^T = K Q^T per 16-key block, seeded with -m
  df32x4 s2[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int kfirst = k0 + 16 * kb;
    const int klast = min(kfirst + 15, c.k_hi - 1);
    const bool any_rem = PATH != DEC_PLAIN && !c.plain && c.pos - kfirst > c.w0;
    const bool any_loc = PATH == DEC_PLAIN || c.plain || c.pos - klast <= c.w0;
    const int key = kfirst + c.r16;
    dh8v kf[NDS];
    if (any_rem && c.pos - key > c.w0) {
      // R_{f(k) - k} (FACT: its in-chunk factor): absolute -> remapped
      // rotation, pairs (ds, ds + NDS/2), in packed fp16 arithmetic on two
      // neighbouring frequencies at a time (the bf16 key values are exact in
      // fp16)
#pragma unroll
      for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const dh2v cr = PATH == DEC_FACT ? tcr[kb][ds][m] : rc[kb][ds][m];
          const dh2v sr = PATH == DEC_FACT ? tsr[kb][ds][m] : rs[kb][ds][m];
          const uint32_t w0 = b.k[kb][ds][m], w1 = b.k[kb][ds + NDS / 2][m];
          const dh2v x0 = {(_Float16)__uint_as_float(w0 << 16),
                           (_Float16)__uint_as_float(w0 & 0xffff0000u)};
          const dh2v x1 = {(_Float16)__uint_as_float(w1 << 16),
                           (_Float16)__uint_as_float(w1 & 0xffff0000u)};
          const dh2v y0 = x0 * cr - x1 * sr;
          const dh2v y1 = x0 * sr + x1 * cr;
          kf[ds][2 * m] = y0[0];
          kf[ds][2 * m + 1] = y0[1];
          kf[ds + NDS / 2][2 * m] = y1[0];
          kf[ds + NDS / 2][2 * m + 1] = y1[1];
        }
    } else {
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) kf[ds] = dec_to_f16(b.k[kb][ds]);
    }
    if (!any_loc) {
      dec_qk<D>(kf, qr, st.negm, s2[kb]);
    } else if (!any_rem) {
      dec_qk<D>(kf, qa, st.negm, s2[kb]);
    } else {
      // block across the window edge: each lane (one key) keeps its fragment
      // for its own route and zeros it for the other, so one accumulation
      // chain adds exactly one product per key
      const bool rem = c.pos - key > c.w0;
      dh8v kl[NDS], krm[NDS];
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const dh8v z = {};
        kl[ds] = rem ? z : kf[ds];
        krm[ds] = rem ? kf[ds] : z;
      }
      df32x4 t;
      dec_qk<D>(kl, qa, st.negm, t);
      dec_qk<D>(krm, qr, t, s2[kb]);
    }
    chk += (s2[kb][0] + s2[kb][1]) + (s2[kb][2] + s2[kb][3]);
    if (klast - kfirst < 15) {  // keys past the range end
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (kfirst + 4 * c.g16 + r >= c.k_hi) s2[kb][r] = -INFINITY;
    }
  }
  // ---- softmax with the lazy reference
  db8v pb;
  float psum = dec_exp(s2, pb);
  const bool need = !(psum <= kDecSumMax) || st.m == -INFINITY;
  if (__any(need)) {
    // move the reference of the queries that need it to their chunk max; a
    // query's scores live in lanes r16 + 16 g, g = 0..3
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mt = fmaxf(mt, s2[kb][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    float nf = need ? 1.f : 0.f;
    nf = fmaxf(nf, __shfl_xor(nf, 16));
    nf = fmaxf(nf, __shfl_xor(nf, 32));
    const bool grow = nf > 0.f && mt > -INFINITY;
    const float delta = grow ? mt : 0.f;
    const float alpha = grow ? (st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(-mt)) : 1.f;
    st.lsum *= alpha;
    if (grow) st.m = (st.m == -INFINITY ? 0.f : st.m) + mt;
    const float nm = st.m == -INFINITY ? 0.f : -st.m;
    st.negm = df32x4{nm, nm, nm, nm};
    // output rows of this lane are queries 4 g16 + r, held as r16 by lane 4 g16 + r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float al = __shfl(alpha, 4 * c.g16 + r);
#pragma unroll
      for (int db = 0; db < NDB; ++db) st.acc[db][r] *= al;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) s2[kb][r] -= delta;
    psum = dec_exp(s2, pb);
  }
  st.lsum += psum;
  // ---- O += P V, the V operand through transpose reads of the LDS stage:
  // lane (g16, r16) addresses row 4 g16 + r16 / 4 (and + 16), dims
  // 16 db + 4 (r16 % 4) .. + 3, i.e. byte 8 (r16 & 1) of chunk
  // 2 db + (r16 & 3) / 2 before the swizzle
  const int row = 4 * c.g16 + (c.r16 >> 2);
  const int sub = 8 * (c.r16 & 1);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int ch = 2 * db + ((c.r16 & 3) >> 1);
    const ds4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) ds4v*)(vb + row * VROW +
                                                  16 * (ch ^ dec_vswz<D>(row)) + sub));
    const ds4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) ds4v*)(vb + (row + 16) * VROW +
                                                  16 * (ch ^ dec_vswz<D>(row + 16)) + sub));
    const db8v vop =
        __builtin_bit_cast(db8v, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    st.acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb, vop, st.acc[db], 0, 0, 0);
  }
}

// Records of the bf16 decode: for (sequence b, KV head g, range s) at
// rec + ((b Hkv + g) S + s) recf floats: (m, l) of each query head of the
// group in the first 2 DEC_RP floats, then the unnormalised O [R][D].
__host__ __device__ inline int dec_recf(int R, int D) { return 2 * DEC_RP + R * D; }

// The outputs of KV head g's query heads for sequence b are NaN (an entry
// outside the caller's bounds, or an operand out of the fp16 range).
template <int D>
__device__ __forceinline__ void dec_write_nan(const DecArgs& a, int b, int g) {
  const int R = a.Hq / a.Hkv;
  const int64_t row0 = (int64_t)b * a.Hq + (int64_t)g * R;
  for (int idx = threadIdx.x; idx < R * D; idx += blockDim.x)
    ((uint16_t*)a.o)[row0 * D + idx] = 0x7fc0;
  if (a.lse && threadIdx.x < R) a.lse[row0 + threadIdx.x] = __builtin_nanf("");
}

// One work unit: KV head g, range s (of nrange) of sequence b. Every thread
// of the workgroup calls it; it returns with the LDS free for the next unit.
template <int D, int PATH>
__device__ __forceinline__ void dec_unit(const DecArgs& a, const DecSeq& sq, int b, int g, int s,
                                         int nrange, const DecLds<D>& sh) {
  using Gm = DecGeom<D>;
  constexpr int NDS = Gm::NDS, NDB = Gm::NDB, HALF = D / 2;
  const int tid = threadIdx.x;
  // the wave index is uniform per wave: say so, so that every range-derived
  // value lives in scalar registers and the route branches are scalar jumps;
  // matrix instructions then never run under a partial EXEC mask
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int R = a.Hq / a.Hkv, h0 = g * R;

  DecCtx c;
  const int k_lo = s * a.kps;
  c.k_hi = min(k_lo + a.kps, sq.pos + 1);
  c.rstride = (int64_t)a.Hkv * D;
  c.kbase = (const uint16_t*)sq.kc + (int64_t)g * D + 8 * g16;
  c.vbase = (const uint16_t*)sq.vc + (int64_t)g * D;
  c.pos = sq.pos;
  c.w0 = a.w0;
  c.G = sq.G;
  c.plain = a.plain || sq.G == 1;
  c.cont = a.cont;
  c.fk_rel = sq.fk_rel;
  c.fpos = remap_pos(sq.pos, sq.G, a.cont);
  c.lane = lane;
  c.g16 = g16;
  c.r16 = r16;
  constexpr int kstep = DEC_CHUNK * DEC_NW;
  int k0 = k_lo + DEC_CHUNK * wave;
  const bool active = k0 < c.k_hi;  // the range holds a chunk for this wave
  uint8_t* sA = sh.vA + wave * Gm::VBYTES;
  uint8_t* sB = sh.vB + wave * Gm::VBYTES;
  DecBuf<D> bA, bB;
  // the wave's first chunk is in flight during the prologue
  if (active) {
    dec_issue_k<D>(c, k0, bA);
    dec_issue_v<D>(c, k0, sA);
  }

  // ---- prologue: frequencies, the group's raw query, operand tables. The
  // tables read once go to the second V stages (free until the key loop).
  if (tid < HALF) sh.w2pi[tid] = a.fr.w(tid) * kInvTwoPi;
  if (tid == 0) sh.flag[0] = 0;
  {
    const uint16_t* xq = (const uint16_t*)sq.xq + (int64_t)h0 * D;
    for (int idx = tid; idx < 8 * D; idx += blockDim.x)
      sh.qraw[idx] = idx / D < R ? bf16_bits_to_f32(xq[idx]) * a.scale_log2 : 0.f;
  }
  __syncthreads();
  _Float16* pqa = (_Float16*)sh.vB;  // [16][D] query at pos
  _Float16* pq2 = pqa + 16 * D;                  // GEN: [16][D] query at f(pos);
                                                 // FACT: [2][32][HALF] in-chunk cos, sin
  for (int idx = tid; idx < 16 * HALF; idx += blockDim.x) {
    const int h = idx / HALF, i = idx % HALF;
    float y0 = 0.f, y1 = 0.f, z0 = 0.f, z1 = 0.f;
    if (h < R) {
      const float x0 = sh.qraw[h * D + i], x1 = sh.qraw[h * D + i + HALF];
      float cs, sn;
      rope_cs_turns((double)sq.pos, sh.w2pi[i], cs, sn);
      y0 = x0 * cs - x1 * sn;
      y1 = x0 * sn + x1 * cs;
      if (PATH == DEC_GEN) {
        rope_cs_turns(c.fpos, sh.w2pi[i], cs, sn);
        z0 = x0 * cs - x1 * sn;
        z1 = x0 * sn + x1 * cs;
      }
    }
    pqa[h * D + i] = (_Float16)y0;
    pqa[h * D + i + HALF] = (_Float16)y1;
    if (PATH == DEC_GEN) {
      pq2[h * D + i] = (_Float16)z0;
      pq2[h * D + i + HALF] = (_Float16)z1;
    }
  }
  if (PATH == DEC_FACT) {
    // in-chunk factor R_{f(i) - i}, i = 0..31 (f(k0 + i) - f(k0) = f(i) as
    // G divides k0, or the map is linear)
    for (int idx = tid; idx < 32 * HALF; idx += blockDim.x) {
      const int i = idx / HALF, f = idx % HALF;
      const double din = a.cont ? (double)i * sq.fk_rel : (double)(i / sq.G - i);
      float cs, sn;
      rope_cs_turns(din, sh.w2pi[f], cs, sn);
      pq2[idx] = (_Float16)cs;
      pq2[32 * HALF + idx] = (_Float16)sn;
    }
  }
  if (PATH == DEC_GEN) {
    // R_{c16} for both values of c16 = f(k + 16) - f(k) - 16 (continuous
    // map: 16 (1 / G - 1) in both)
    _Float16* tt = (_Float16*)sh.cs;  // [2 steps][cos, sin][HALF]
    for (int idx = tid; idx < 2 * HALF; idx += blockDim.x) {
      const int t = idx / HALF, f = idx % HALF;
      const double c16 = a.cont ? 16.0 * sq.fk_rel : (double)(16 / sq.G + t - 16);
      float cs, sn;
      rope_cs_turns(c16, sh.w2pi[f], cs, sn);
      tt[2 * t * HALF + f] = (_Float16)cs;
      tt[(2 * t + 1) * HALF + f] = (_Float16)sn;
    }
  }
  __syncthreads();
  dh8v qa[NDS], qr[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    qa[ds] = *(const dh8v*)(pqa + r16 * D + 32 * ds + 8 * g16);
    qr[ds] = PATH == DEC_GEN ? *(const dh8v*)(pq2 + r16 * D + 32 * ds + 8 * g16) : dh8v{};
  }
  dh2v tcr[2][NDS / 2][4], tsr[2][NDS / 2][4];
  if (PATH == DEC_FACT) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ds = 0; ds < NDS / 2; ++ds) {
        const int off = (16 * kb + r16) * HALF + 32 * ds + 8 * g16;
        const du32x4 cv = *(const du32x4*)(pq2 + off);
        const du32x4 sv = *(const du32x4*)(pq2 + 32 * HALF + off);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          // (the element is copied first: a bit cast of a vector element
          // expression reads element 0 whatever the index)
          const uint32_t cw = cv[m], sw = sv[m];
          tcr[kb][ds][m] = __builtin_bit_cast(dh2v, cw);
          tsr[kb][ds][m] = __builtin_bit_cast(dh2v, sw);
        }
      }
  }
  __syncthreads();  // the second V stages are free from here on

  DecState<D> st;
#pragma unroll
  for (int db = 0; db < NDB; ++db) st.acc[db] = df32x4{0.f, 0.f, 0.f, 0.f};
  st.negm = df32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.lsum = 0.f;
  float chk = 0.f;

  // chunk n + 1 (K in registers, V in the other LDS stage) is in flight
  // while chunk n is computed. The next chunk is always issued: its keys are
  // clamped to the range, so past the end it re-reads the last key (from L2)
  // and the loads need no branch.
  if (active) {
    for (;;) {
      dec_issue_k<D>(c, k0 + kstep, bB);
      dec_issue_v<D>(c, k0 + kstep, sB);
      __builtin_amdgcn_sched_barrier(0);  // all of the next chunk's loads go out first
      dec_chunk<D, PATH>(c, k0, bA, qa, qr, tcr, tsr, sh, wave, sA, st, chk);
      if (k0 + kstep >= c.k_hi) break;
      dec_issue_k<D>(c, k0 + 2 * kstep, bA);
      dec_issue_v<D>(c, k0 + 2 * kstep, sA);
      __builtin_amdgcn_sched_barrier(0);
      dec_chunk<D, PATH>(c, k0 + kstep, bB, qa, qr, tcr, tsr, sh, wave, sB, st, chk);
      if (k0 + 2 * kstep >= c.k_hi) break;
      k0 += 2 * kstep;
    }
  }
  // no transfer into the LDS stages may outlive the loop
  __builtin_amdgcn_s_waitcnt(0);
  if (__any(!(chk - chk == 0.f))) {  // chk is inf or NaN
    if (lane == 0) atomicOr(&sh.flag[0], 1);
  }
  __syncthreads();  // every wave is past its V stages

  // ---- merge the waves' states through LDS into the range's record
  float* red = (float*)sh.vA;
  float* red_m = red;                  // [NW][16]
  float* red_l = red + DEC_NW * 16;    // [NW][16]
  float* red_a = red + 2 * DEC_NW * 16;  // [NW][R][D]
  {
    float lt = st.lsum + __shfl_xor(st.lsum, 16);
    lt += __shfl_xor(lt, 32);
    if (g16 == 0) {
      red_m[wave * 16 + r16] = st.m;
      red_l[wave * 16 + r16] = lt;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = 4 * g16 + r;
      if (q < R) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) red_a[(wave * R + q) * D + 16 * db + r16] = st.acc[db][r];
      }
    }
  }
  __syncthreads();
  const int recf = dec_recf(R, D);
  float* rec0 = a.rec + ((int64_t)b * a.Hkv + g) * a.S * recf;
  {
    float* rec = rec0 + (int64_t)s * recf;
    const bool bad = sh.flag[0] != 0;
    for (int idx = tid; idx < R * D; idx += blockDim.x) {
      const int h = idx / D, dd = idx % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < DEC_NW; ++w) M = fmaxf(M, red_m[w * 16 + h]);
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < DEC_NW; ++w) {
        const float mw = red_m[w * 16 + h];
        const float sc = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L += red_l[w * 16 + h] * sc;
        A += red_a[(w * R + h) * D + dd] * sc;
      }
      rec[2 * DEC_RP + idx] = A;
      if (dd == 0) {
        rec[2 * h] = M;
        rec[2 * h + 1] = bad ? __builtin_nanf("") : L;
      }
    }
  }
  // ---- release the record, take the ticket; the last range merges
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  int* ticket = a.tickets + (int64_t)b * a.Hkv + g;
  if (tid == 0) sh.flag[1] = atomicAdd(ticket, 1) == nrange - 1;
  __syncthreads();
  if (!sh.flag[1]) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  {
    // thread = (group of ranges grp, 4 consecutive elements e4 of the
    // [R][D] output); batches of 16 ranges, all loads issued before use
    const int e4n = R * D / 4;
    const int ng = blockDim.x / e4n;  // e4n divides 256 for R in {1, 2, 4, 8}
    const int grp = tid / e4n, e4 = tid % e4n;
    const int h = 4 * e4 / D;
    float M = -INFINITY, L = 0.f;
    df32x4 A = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = grp; s0 < nrange; s0 += 16 * ng) {
      float2 ml[16];
      df32x4 av[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int sj = s0 + j * ng;
        const float* r = rec0 + (int64_t)(sj < nrange ? sj : s0) * recf;
        ml[j] = *(const float2*)(r + 2 * h);
        av[j] = *(const df32x4*)(r + 2 * DEC_RP + 4 * e4);
        if (sj >= nrange) ml[j].x = -INFINITY;
      }
      float mb = M;
#pragma unroll
      for (int j = 0; j < 16; ++j) mb = fmaxf(mb, ml[j].x);
      const float sc = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - mb);
      L *= sc;
      A *= sc;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float w = ml[j].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[j].x - mb);
        L += w * ml[j].y;
        A += w * av[j];
      }
      M = mb;
    }
    // combine the groups through LDS (the records' merge scratch is free)
    __syncthreads();
    float* gm = red;                  // [ng][e4n]
    float* gl = red + 256;            // [ng][e4n]
    df32x4* ga = (df32x4*)(red + 512);  // [ng][e4n]
    if (grp < ng) {
      gm[tid] = M;
      gl[tid] = L;
      ga[tid] = A;
    }
    __syncthreads();
    if (tid < e4n) {
      float Mt = -INFINITY;
      for (int q = 0; q < ng; ++q) Mt = fmaxf(Mt, gm[q * e4n + e4]);
      float Lt = 0.f;
      df32x4 At = {0.f, 0.f, 0.f, 0.f};
      for (int q = 0; q < ng; ++q) {
        const float mq = gm[q * e4n + e4];
        const float w = mq == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mq - Mt);
        Lt += w * gl[q * e4n + e4];
        At += w * ga[q * e4n + e4];
      }
      const int64_t orow = (int64_t)b * a.Hq + h0 + h;
      const int dd = 4 * e4 - h * D;
      const float inv = 1.f / Lt;
      const uint32_t lo = (uint32_t)f32_to_bf16_bits(At[0] * inv) |
                          ((uint32_t)f32_to_bf16_bits(At[1] * inv) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_bits(At[2] * inv) |
                          ((uint32_t)f32_to_bf16_bits(At[3] * inv) << 16);
      *(uint2*)((uint16_t*)a.o + orow * D + dd) = make_uint2(lo, hi);
      if (a.lse && dd == 0) a.lse[orow] = (Mt + __log2f(Lt)) * 0.69314718055994530942f;
    }
  }
  if (tid == 0) atomicExch(ticket, 0);  // every range of this head has arrived: ready for the next call
  __syncthreads();
}

// Single sequence: workgroup (range s, KV head g) = blockIdx (s Hkv + g), so
// the workgroups running together cover every head of the same key rows.
template <int D, int PATH>
__global__ void __launch_bounds__(256, 2) decode_bf16_kernel(DecArgs a) {
  const DecLds<D> sh = dec_lds<D>();
  const int g = blockIdx.x % a.Hkv, s = blockIdx.x / a.Hkv;
  const DecSeq sq = dec_seq<false>(a, 0, D, 2);
  dec_unit<D, PATH>(a, sq, 0, g, s, a.S, sh);
}

// Batch: a fixed grid of workgroups walks the work list the plan kernel
// built (unit u = (entry u / Hkv of the list, KV head u % Hkv); the list
// holds the ranges s * kps <= pos_b of every valid sequence b, base[b] ..
// base[b + 1] - 1, and one entry per invalid sequence), round robin, so the
// work spreads evenly over the CUs whatever the mix of lengths.
template <int D>
__global__ void __launch_bounds__(256, 2) decode_bf16_batch_kernel(DecArgs a, const int* base,
                                                                   int B) {
  const DecLds<D> sh = dec_lds<D>();
  const int units = base[B] * a.Hkv;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int item = u / a.Hkv, g = u % a.Hkv;
    int lo = 0, hi = B - 1;  // the sequence b with base[b] <= item < base[b + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (base[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const DecSeq sq = dec_seq<true>(a, lo, D, 2);
    if (!sq.ok) {  // an entry outside the caller's bounds reads nothing
      dec_write_nan<D>(a, lo, g);
      continue;
    }
    // one path (a second would not fit the registers): the general
    // correction, skipped at run time for plain mode and G = 1
    dec_unit<D, DEC_GEN>(a, sq, lo, g, item - base[lo], (sq.pos + a.kps) / a.kps, sh);
  }
}

// Ranges of batch entry b that hold keys (s * kps <= pos); an entry the
// kernels skip takes one list entry (which writes its NaN outputs).
__device__ __forceinline__ int dec_batch_nsplit(const DecArgs& a, int b) {
  const DecSeq sq = dec_seq<true>(a, b, 0, 0);
  return sq.ok ? (sq.pos + a.kps) / a.kps : 1;
}

// Work list of a batched decode: base[b] = number of list entries of the
// entries before b; base[B] = their total. One workgroup.
__global__ void __launch_bounds__(1024) decode_batch_plan_kernel(DecArgs a, int* base, int B) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int per = (B + 1023) / 1024;
  const int b0 = min(tid * per, B), b1 = min(b0 + per, B);
  int sum = 0;
  for (int b = b0; b < b1; ++b) sum += dec_batch_nsplit(a, b);
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = tid ? part[tid - 1] : 0;
  for (int b = b0; b < b1; ++b) {
    base[b] = run;
    run += dec_batch_nsplit(a, b);
  }
  if (tid == 1023) base[B] = part[1023];
}

// Zero fill (the arrival tickets of a fresh workspace): a kernel rather than
// a memset, so the call is safe to record in a graph.
__global__ void __launch_bounds__(256) dec_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = 0u;
}

// float32 merge of the split partials of one query head with LSE weights:
// workgroup (head h, 16 output dims), thread (split group g of 16, dim):
// each thread takes the splits s = g, g + 16, ... sixteen at a time, all of a
// batch's loads issued before any is used (one memory round trip for up to
// 256 splits), folds them with a running maximum, and the 16 groups are
// combined through LDS.
template <bool F32, int D, bool BATCH>
__global__ void __launch_bounds__(256) decode_merge_kernel(DecArgs a) {
  __shared__ float rm[256], rl[256], ra[256];
  const int h = blockIdx.x, d0 = 16 * blockIdx.y, tid = threadIdx.x;
  const int dd = tid & 15, grp = tid >> 4;
  const int b = blockIdx.z;
  const DecSeq sq = dec_seq<BATCH>(a, b, D, F32 ? 4 : 2);
  const int64_t orow = (int64_t)b * a.Hq + h;  // output row of (sequence, head)
  if (!sq.ok) {  // a skipped batch entry: NaN marks it (uniform exit)
    if (grp == 0) {
      if constexpr (F32) ((float*)a.o)[orow * D + d0 + dd] = __builtin_nanf("");
      else ((uint16_t*)a.o)[orow * D + d0 + dd] = 0x7fc0;
      if (a.lse && d0 + dd == 0) a.lse[orow] = __builtin_nanf("");
    }
    return;
  }
  // splits that hold keys of this sequence: s * kps <= pos
  const int S = BATCH ? (sq.pos + a.kps) / a.kps : a.S;
  const float* pp = sq.part + (int64_t)h * a.S * (D + 2);
  float M = -INFINITY, L = 0.f, A = 0.f;
  for (int s0 = grp; s0 < S; s0 += 256) {
    float ms[16], ls[16], as[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int s = s0 + 16 * j;
      const float* q = pp + (int64_t)(s < S ? s : 0) * (D + 2);
      ms[j] = s < S ? q[0] : -INFINITY;
      ls[j] = s < S ? q[1] : 0.f;
      as[j] = s < S ? q[2 + d0 + dd] : 0.f;
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < 16; ++j) mb = fmaxf(mb, ms[j]);
    if (mb > -INFINITY) {  // -inf partials (no keys) carry no weight
      const float sc = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - mb);
      L *= sc;
      A *= sc;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float w = ms[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[j] - mb);
        L += w * ls[j];
        A += w * as[j];
      }
      M = mb;
    }
  }
  rm[tid] = M;
  rl[tid] = L;
  ra[tid] = A;
  __syncthreads();
  if (grp == 0) {
    float Mt = -INFINITY;
#pragma unroll
    for (int g = 0; g < 16; ++g) Mt = fmaxf(Mt, rm[16 * g + dd]);
    float Lt = 0.f, At = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const float mg = rm[16 * g + dd];
      const float w = mg == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mg - Mt);
      Lt += w * rl[16 * g + dd];
      At += w * ra[16 * g + dd];
    }
    const float out = At / Lt;
    if constexpr (F32) ((float*)a.o)[orow * D + d0 + dd] = out;
    else ((uint16_t*)a.o)[orow * D + d0 + dd] = f32_to_bf16_bits(out);
    if (a.lse && d0 + dd == 0) a.lse[orow] = (Mt + __log2f(Lt)) * 0.69314718055994530942f;
  }
}


template <int D, bool BATCH>
static void launch_decode_f32(int R, int B, hipStream_t st, const DecArgs& a) {
  const dim3 grid(a.S, a.Hkv, B);
  switch (R) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<true, D, 1, BATCH>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<true, D, 2, BATCH>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<true, D, 4, BATCH>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((decode_split_kernel<true, D, 8, BATCH>), grid, dim3(256), 0, st, a); break;
  }
  hipLaunchKernelGGL((decode_merge_kernel<true, D, BATCH>), dim3(a.Hq, D / 16, B), dim3(256), 0,
                     st, a);
}

template <int D>
static void launch_decode_bf16(int path, hipStream_t st, const DecArgs& a) {
  const dim3 grid((unsigned)(a.S * a.Hkv));
  if (path == DEC_PLAIN)
    hipLaunchKernelGGL((decode_bf16_kernel<D, DEC_PLAIN>), grid, dim3(256), 0, st, a);
  else if (path == DEC_FACT)
    hipLaunchKernelGGL((decode_bf16_kernel<D, DEC_FACT>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((decode_bf16_kernel<D, DEC_GEN>), grid, dim3(256), 0, st, a);
}

static DecArgs decode_args(const void* xq, const void* kc, const void* vc, void* o, float* lse,
                           int Hq, int Hkv, int64_t w0, float scale, const RopeFreqs& fr,
                           int plain, int cont, int* tickets, float* part) {
  DecArgs a;
  a.xq = xq;
  a.kc = kc;
  a.vc = vc;
  a.part = part;
  a.rec = part;
  a.tickets = tickets;
  a.o = o;
  a.lse = lse;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.w0 = (int)w0;
  a.plain = plain;
  a.cont = cont;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.fr = fr;
  a.pos = 0;
  a.G = 1;
  a.fk_rel = 0.0;
  a.bpos = nullptr;
  a.bstart = nullptr;
  a.max_keys = 0;
  a.cap_rows = 0;
  a.w_pre = 1;
  return a;
}

hipError_t launch_decode(const void* xq, const void* kc, const void* vc, void* o, float* lse,
                         int64_t pos, int Hq, int Hkv, int d, int64_t w0, int64_t G, float scale,
                         const RopeFreqs& fr, int plain, int cont, int is_f32, int kps,
                         int* tickets, float* part, hipStream_t st) {
  DecArgs a = decode_args(xq, kc, vc, o, lse, Hq, Hkv, w0, scale, fr, plain, cont, tickets, part);
  a.pos = (int)pos;
  a.G = (int)G;
  a.fk_rel = 1.0 / (double)G - 1.0;
  const int keys = (int)pos + 1;
  a.S = (keys + kps - 1) / kps;  // no empty split
  a.kps = kps;
  if (is_f32) {
    if (d == 64) launch_decode_f32<64, false>(Hq / Hkv, 1, st, a);
    else launch_decode_f32<128, false>(Hq / Hkv, 1, st, a);
  } else {
    const int path = (plain || G == 1) ? DEC_PLAIN : (cont || 32 % G == 0) ? DEC_FACT : DEC_GEN;
    if (d == 64) launch_decode_bf16<64>(path, st, a);
    else launch_decode_bf16<128>(path, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_batch(const void* xq, const void* kc, const void* vc, void* o, float* lse,
                               const int32_t* positions, const int32_t* starts, int B,
                               int64_t max_keys, int64_t cap_rows, int Hq, int Hkv, int d,
                               int64_t w0, int64_t w_pre, float scale, const RopeFreqs& fr,
                               int plain, int cont, int is_f32, int splits, int kps, int* tickets,
                               float* part, int* base, int grid_wg, hipStream_t st) {
  DecArgs a = decode_args(xq, kc, vc, o, lse, Hq, Hkv, w0, scale, fr, plain, cont, tickets, part);
  a.bpos = positions;
  a.bstart = starts;
  a.max_keys = (int)max_keys;
  a.cap_rows = cap_rows;
  a.w_pre = w_pre;
  a.S = splits;
  a.kps = kps;
  if (is_f32) {
    if (d == 64) launch_decode_f32<64, true>(Hq / Hkv, B, st, a);
    else launch_decode_f32<128, true>(Hq / Hkv, B, st, a);
  } else {
    hipLaunchKernelGGL(decode_batch_plan_kernel, dim3(1), dim3(1024), 0, st, a, base, B);
    if (d == 64)
      hipLaunchKernelGGL((decode_bf16_batch_kernel<64>), dim3(grid_wg), dim3(256), 0, st, a,
                         (const int*)base, B);
    else
      hipLaunchKernelGGL((decode_bf16_batch_kernel<128>), dim3(grid_wg), dim3(256), 0, st, a,
                         (const int*)base, B);
  }
  return hipGetLastError();
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const size_t want = (n + 255) / 256;
  const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(dec_zero_kernel, dim3(blocks), dim3(256), 0, st, (uint32_t*)p, n);
  return hipGetLastError();
}

}  // namespace jl
