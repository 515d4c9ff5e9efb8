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
// Split-K: each split streams keys [s*n, (s+1)*n) of one KV head once, for
// all Hq/Hkv query heads of the group, and leaves a partial (max, sum,
// unnormalised accumulator) per query head; a second kernel merges the splits
// with LSE weights. HBM traffic is the K and V rows of keys 0..pos read once.
// The bf16 kernel runs one split per wave (a workgroup covers four KV heads
// of one key range); the float32 kernel one split per workgroup.
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
// bf16 path: one wave per split, both products on the matrix cores.
//
// Per 64-key chunk a wave loads K (as the A operand of S^T = K Q^T, fp16,
// 16x16x32 MFMAs: lane = one key, 8 consecutive dims) and V (row-major into a
// wave-private LDS region). Remote keys are corrected in-lane: the pairs
// (i, i + D/2) of a key sit in d-steps ds and ds + D/64 of the same lane. The
// S^T tile gives each lane one query (lane % 16) and four keys per 16-key
// block, which is exactly the A operand of O = P V for two consecutive
// blocks; the V operand (8 keys at one dim per lane) comes from LDS with the
// transpose read ds_read_b64_tr_b16: within 16 lanes, lane i receives element
// i % 4 of the 8-byte rows addressed by lanes i / 4 + 4t, t = 0..3, so lanes
// pointing at V[key_t][4c .. 4c + 3] deliver V[key_t][own dim] for 4 keys.
// Query heads are padded to the 16 MFMA columns with zeros.
//
// Softmax: the query operand carries scale * log2(e) and the score
// accumulator starts at -m, m a per-split reference that moves only when a
// lane's sum of bf16-rounded p over the chunk exceeds 2^8 (or on the first
// scores), so the common chunk needs no row max and no cross-lane exchange.
// ---------------------------------------------------------------------------
typedef _Float16 dh8v __attribute__((ext_vector_type(8)));
typedef _Float16 dh2v __attribute__((ext_vector_type(2)));
typedef __bf16 db8v __attribute__((ext_vector_type(8)));
typedef __bf16 db2v __attribute__((ext_vector_type(2)));
typedef short ds4v __attribute__((ext_vector_type(4)));
typedef float df32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t du32x4 __attribute__((ext_vector_type(4)));

constexpr int DEC_CHUNK = 32;  // keys per chunk; two chunks are in flight per wave
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

// Per-wave constants of the key loop (all wave-uniform except the lane ids).
struct DecCtx {
  const uint16_t* kbase;  // this lane's K slice: head, dims 8 * g16 ..
  const uint16_t* vbase;  // the head's V row 0
  int64_t rstride;        // elements between consecutive keys
  int pos, w0, G, plain, correct, k_hi;
  int cont;       // remote map x / G (real) instead of floor(x / G)
  double fk_rel;  // with cont: f(k) - k = k * fk_rel
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
// fp16 range), optionally rotated by the remote correction first.
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
    // keys past the split end load the last key (finite data, masked later)
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

template <int D>
__device__ __forceinline__ void dec_chunk(const DecCtx& c, int k0, const DecBuf<D>& b,
                                          const dh8v (&qa)[D / 32], const dh8v (&qr)[D / 32],
                                          const double* w2pi, const uint8_t* vb,
                                          DecState<D>& st, bool step16,
                                          const dh2v (&cst)[D / 64][4],
                                          const dh2v (&sst)[D / 64][4], float& chk) {
  using G = DecGeom<D>;
  constexpr int NDS = G::NDS, NDB = G::NDB, VROW = G::VROW;
  // ---- cos / sin of the correction R_{f(k) - k} of the lane's key in both
  // blocks (pairs (ds, ds + NDS/2), frequencies 32 ds + 8 g16 + j), as fp16
  // pairs of neighbouring frequencies (j, j + 1), the layout of the key
  // fragments. They depend on the key index only, so they are computed
  // before the chunk's data is first touched, i.e. while its loads (and the
  // next chunk's) are still in flight.
  dh2v rc[2][NDS / 2][4], rs[2][NDS / 2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = k0 + 16 * kb + c.r16;
    if (c.correct && c.pos - (k0 + 16 * kb) > c.w0) {  // the block has remote keys
      if (kb == 1 && step16) {
        // key + 16 (block 0 is remote too): the angle moves by a fixed step,
        // R_{d + c16} = R_d R_{c16}
#pragma unroll
        for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            rc[1][ds][m] = rc[0][ds][m] * cst[ds][m] - rs[0][ds][m] * sst[ds][m];
            rs[1][ds][m] = rs[0][ds][m] * cst[ds][m] + rc[0][ds][m] * sst[ds][m];
          }
      } else {
        const double delta = c.cont ? (double)key * c.fk_rel : (double)(key / c.G - key);
#pragma unroll
        for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            float c0, s0, c1, s1;
            rope_cs_turns(delta, w2pi[32 * ds + 8 * c.g16 + 2 * m], c0, s0);
            rope_cs_turns(delta, w2pi[32 * ds + 8 * c.g16 + 2 * m + 1], c1, s1);
            rc[kb][ds][m] = dh2v{(_Float16)c0, (_Float16)c1};
            rs[kb][ds][m] = dh2v{(_Float16)s0, (_Float16)s1};
          }
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
    const bool any_rem = !c.plain && c.pos - kfirst > c.w0;
    const bool any_loc = c.plain || c.pos - klast <= c.w0;
    const int key = kfirst + c.r16;
    dh8v kf[NDS];
    if (c.correct && c.pos - key > c.w0) {
      // R_{f(k) - k}: absolute -> remapped rotation, pairs (ds, ds + NDS/2),
      // in packed fp16 arithmetic on two neighbouring frequencies at a time
      // (the bf16 key values are exact in fp16)
#pragma unroll
      for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t w0 = b.k[kb][ds][m], w1 = b.k[kb][ds + NDS / 2][m];
          const dh2v x0 = {(_Float16)__uint_as_float(w0 << 16),
                           (_Float16)__uint_as_float(w0 & 0xffff0000u)};
          const dh2v x1 = {(_Float16)__uint_as_float(w1 << 16),
                           (_Float16)__uint_as_float(w1 & 0xffff0000u)};
          const dh2v y0 = x0 * rc[kb][ds][m] - x1 * rs[kb][ds][m];
          const dh2v y1 = x0 * rs[kb][ds][m] + x1 * rc[kb][ds][m];
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
    // raw scores of an fp16 operand out of range are not finite: their sum
    // carries that to the end of the split
    chk += (s2[kb][0] + s2[kb][1]) + (s2[kb][2] + s2[kb][3]);
    if (klast - kfirst < 15) {  // keys past the split end
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

// One work unit of the bf16 decode for one wave: keys [s kps, (s + 1) kps)
// of KV head kvh of sequence sq, leaving the partial of each query head of
// the group. vA / vB: this wave's two V stages.
// cos / sin tables a workgroup computes once for the rotations shared by all
// of its lanes: [0][i] of pos * omega_i, [1][i] of f(pos) * omega_i (the
// query at the absolute and the remapped position), [2][i] of c16 * omega_i
// (the step between a chunk's two 16-key blocks). One angle per thread.
template <int D>
__device__ __forceinline__ void dec_tables(const DecArgs& a, const DecSeq& sq, bool step16,
                                           const double* w2pi_s, float2 (*tab)[D / 2]) {
  const int i = threadIdx.x;
  if (i < D / 2) {
    const double w = w2pi_s[i];
    float c, s;
    rope_cs_turns((double)sq.pos, w, c, s);
    tab[0][i] = make_float2(c, s);
    if (!a.plain) {
      rope_cs_turns(remap_pos(sq.pos, sq.G, a.cont), w, c, s);
      tab[1][i] = make_float2(c, s);
    }
    if (step16) {
      rope_cs_turns(a.cont ? 16.0 * sq.fk_rel : (double)(16 / sq.G - 16), w, c, s);
      tab[2][i] = make_float2(c, s);
    }
  }
}

// Whether the second 16-key block of a chunk takes its cos / sin from the
// first by one rotation R_{c16}: with G dividing 16 (floor map) or the
// continuous map, f(k) - k moves by the same c16 from key k to key k + 16.
__device__ __forceinline__ bool dec_step16(const DecArgs& a, const DecSeq& sq) {
  return !a.plain && sq.G > 1 && (a.cont || 16 % sq.G == 0);
}

template <int D, bool STEP16>
__device__ __forceinline__ void dec_unit(const DecArgs& a, const DecSeq& sq, int s, int kvh,
                                         const double* w2pi_s, const float2 (*tab)[D / 2],
                                         uint8_t* sA, uint8_t* sB) {
  using G = DecGeom<D>;
  constexpr int NDS = G::NDS, NDB = G::NDB;
  const int lane = threadIdx.x & 63;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int R = a.Hq / a.Hkv, h0 = kvh * R;
  const uint16_t* xq = (const uint16_t*)sq.xq;
  const uint16_t* kc = (const uint16_t*)sq.kc;
  const uint16_t* vc = (const uint16_t*)sq.vc;

  const int k_lo = s * a.kps;
  DecCtx c;
  c.k_hi = min(k_lo + a.kps, sq.pos + 1);
  c.rstride = (int64_t)a.Hkv * D;
  c.kbase = kc + (int64_t)kvh * D + 8 * g16;
  c.vbase = vc + (int64_t)kvh * D;
  c.pos = sq.pos;
  c.w0 = a.w0;
  c.G = sq.G;
  c.cont = a.cont;
  c.fk_rel = sq.fk_rel;
  c.plain = a.plain;
  c.correct = !a.plain && sq.G > 1;
  c.lane = lane;
  c.g16 = g16;
  c.r16 = r16;

  // the first chunk is in flight while the query operands and tables are
  // computed
  DecBuf<D> bA, bB;
  int k0 = k_lo;
  dec_issue_k<D>(c, k0, bA);
  dec_issue_v<D>(c, k0, sA);

  // query operands (B of S^T = K Q^T): lane holds dims 32 ds + 8 g16 + j of
  // query head r16, rotated at pos (qa) and at f(pos) (qr), times scale*log2 e
  dh8v qa[NDS], qr[NDS];
  {
    // the lane's dims 32 ds + 8 g16 .. + 8 and their partners + D/2, as
    // 16-byte loads of a valid row (head r16 clamped), zeroed past R heads
    const bool qv = r16 < R;
    const uint16_t* qp = xq + (int64_t)(h0 + (qv ? r16 : 0)) * D;
    du32x4 raw0[NDS / 2], raw1[NDS / 2];
#pragma unroll
    for (int ds = 0; ds < NDS / 2; ++ds) {
      raw0[ds] = *(const du32x4*)(qp + 32 * ds + 8 * g16);
      raw1[ds] = *(const du32x4*)(qp + 32 * ds + 8 * g16 + D / 2);
    }
#pragma unroll
    for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 32 * ds + 8 * g16 + j;
        const float x0 = qv ? bf16_lane(raw0[ds], j) : 0.f;
        const float x1 = qv ? bf16_lane(raw1[ds], j) : 0.f;
        const float2 ta = tab[0][i];
        qa[ds][j] = (_Float16)((x0 * ta.x - x1 * ta.y) * a.scale_log2);
        qa[ds + NDS / 2][j] = (_Float16)((x0 * ta.y + x1 * ta.x) * a.scale_log2);
        if (!a.plain) {  // plain mode has no remapped route
          const float2 tr = tab[1][i];
          qr[ds][j] = (_Float16)((x0 * tr.x - x1 * tr.y) * a.scale_log2);
          qr[ds + NDS / 2][j] = (_Float16)((x0 * tr.y + x1 * tr.x) * a.scale_log2);
        } else {
          qr[ds][j] = qr[ds + NDS / 2][j] = (_Float16)0.f;
        }
      }
  }
  // R_{c16} between a chunk's two 16-key blocks (see dec_step16), as fp16
  // pairs of neighbouring frequencies
  const bool step16 = STEP16 && dec_step16(a, sq);
  dh2v cst[NDS / 2][4], sst[NDS / 2][4];
  if (step16) {
#pragma unroll
    for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float2 t0 = tab[2][32 * ds + 8 * g16 + 2 * m];
        const float2 t1 = tab[2][32 * ds + 8 * g16 + 2 * m + 1];
        cst[ds][m] = dh2v{(_Float16)t0.x, (_Float16)t1.x};
        sst[ds][m] = dh2v{(_Float16)t0.y, (_Float16)t1.y};
      }
  }

  DecState<D> st;
#pragma unroll
  for (int db = 0; db < NDB; ++db) st.acc[db] = df32x4{0.f, 0.f, 0.f, 0.f};
  st.negm = df32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.lsum = 0.f;
  float chk = 0.f;

  // chunk i + 1 (K in registers, V in the other LDS stage) is in flight
  // while chunk i is computed. The next chunk is always issued: its keys are
  // clamped to the split, so past the end it re-reads the last key (from L2)
  // and the loads need no branch.
  for (;;) {
    dec_issue_k<D>(c, k0 + DEC_CHUNK, bB);
    dec_issue_v<D>(c, k0 + DEC_CHUNK, sB);
    __builtin_amdgcn_sched_barrier(0);  // all of the next chunk's loads go out first
    dec_chunk<D>(c, k0, bA, qa, qr, w2pi_s, sA, st, step16, cst, sst, chk);
    if (k0 + DEC_CHUNK >= c.k_hi) break;
    dec_issue_k<D>(c, k0 + 2 * DEC_CHUNK, bA);
    dec_issue_v<D>(c, k0 + 2 * DEC_CHUNK, sA);
    __builtin_amdgcn_sched_barrier(0);
    dec_chunk<D>(c, k0 + DEC_CHUNK, bB, qa, qr, w2pi_s, sB, st, step16, cst, sst, chk);
    if (k0 + 2 * DEC_CHUNK >= c.k_hi) break;
    k0 += 2 * DEC_CHUNK;
  }
  // no transfer into these LDS stages may outlive the unit
  __builtin_amdgcn_s_waitcnt(0);
  const float m = st.m, lsum = st.lsum;
  df32x4 (&acc)[NDB] = st.acc;
  // ---- split partial: m (log2 domain), l, unnormalised O for each query head
  float lt = lsum + __shfl_xor(lsum, 16);
  lt += __shfl_xor(lt, 32);
  // an operand out of the fp16 range: every query head of this KV head
  // publishes m = +inf and l = NaN, so the merge's weights, and with them the
  // outputs and the LSE, are NaN (a NaN m alone would be skipped by the max)
  const bool bad = __any(!(chk - chk == 0.f));
  if (bad) lt = __builtin_nanf("");
  float* part = sq.part;
  if (g16 == 0 && r16 < R) {
    float* pp = part + ((int64_t)(h0 + r16) * a.S + s) * (D + 2);
    pp[0] = bad ? INFINITY : m;
    pp[1] = lt;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int q = 4 * g16 + r;
    if (q < R) {
      float* pp = part + ((int64_t)(h0 + q) * a.S + s) * (D + 2) + 2;
#pragma unroll
      for (int db = 0; db < NDB; ++db) pp[16 * db + r16] = acc[db][r];
    }
  }
}

// Single sequence: workgroup = one split of four KV heads (wave w: head
// 4 hg + w), so the waves running together read neighbouring head slices of
// the same key rows.
template <int D>
__global__ void __launch_bounds__(256, 2) decode_mfma_kernel(DecArgs a) {
  using G = DecGeom<D>;
  // two V stages per wave, as separate arrays so that reads of one are known
  // not to alias the transfers in flight into the other
  __shared__ __attribute__((aligned(16))) uint8_t vstA[4][G::VBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vstB[4][G::VBYTES];
  __shared__ double w2pi_s[D / 2];
  __shared__ float2 tab_s[3][D / 2];
  // the wave index is uniform per wave: say so, so that every split-derived
  // value (key range, route of a key block) lives in scalar registers and the
  // route branches are scalar jumps; matrix instructions then never run under
  // a partial or empty EXEC mask
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const DecSeq sq = dec_seq<false>(a, 0, D, 2);
  if (tid < D / 2) w2pi_s[tid] = a.fr.w(tid) * kInvTwoPi;
  __syncthreads();
  dec_tables<D>(a, sq, dec_step16(a, sq), w2pi_s, tab_s);
  __syncthreads();
  const int hgroups = (a.Hkv + 3) >> 2;
  const int s = blockIdx.x / hgroups, kvh = (blockIdx.x % hgroups) * 4 + wave;
  if (kvh >= a.Hkv) return;
  dec_unit<D, true>(a, sq, s, kvh, w2pi_s, tab_s, vstA[wave], vstB[wave]);
}

// Batch: a fixed grid of workgroups walks the work list the plan kernel
// built (unit u = (entry of the list, KV-head group); the list holds the
// splits s * kps <= pos_b of every valid sequence b, base[b] .. base[b+1] -
// 1), round robin, so the work spreads evenly over the CUs whatever the mix
// of sequence lengths.
template <int D>
__global__ void __launch_bounds__(256, 2) decode_mfma_batch_kernel(DecArgs a, const int* base,
                                                                   int B) {
  using G = DecGeom<D>;
  __shared__ __attribute__((aligned(16))) uint8_t vstA[4][G::VBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vstB[4][G::VBYTES];
  __shared__ double w2pi_s[D / 2];
  __shared__ float2 tab_s[3][D / 2];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid < D / 2) w2pi_s[tid] = a.fr.w(tid) * kInvTwoPi;
  __syncthreads();
  const int hgroups = (a.Hkv + 3) >> 2;
  const int units = base[B] * hgroups;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    const int item = u / hgroups, kvh = (u % hgroups) * 4 + wave;
    int lo = 0, hi = B - 1;  // the sequence b with base[b] <= item < base[b + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (base[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const DecSeq sq = dec_seq<true>(a, lo, D, 2);
    // this unit's tables (every wave passes both barriers, also the waves
    // past the last KV head)
    __syncthreads();
    dec_tables<D>(a, sq, false, w2pi_s, tab_s);
    __syncthreads();
    if (kvh >= a.Hkv) continue;
    // (the batch kernel has no registers to spare for the step table)
    dec_unit<D, false>(a, sq, item - base[lo], kvh, w2pi_s, tab_s, vstA[wave], vstB[wave]);
  }
}

// Splits of batch entry b that hold keys (s * kps <= pos), 0 for an entry
// the kernels skip.
__device__ __forceinline__ int dec_batch_nsplit(const DecArgs& a, int b) {
  const DecSeq sq = dec_seq<true>(a, b, 0, 0);
  return sq.ok ? (sq.pos + a.kps) / a.kps : 0;
}

// Work list of a batched decode: base[b] = number of splits of the entries
// before b; base[B] = their total. One workgroup.
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

// Merge of the split partials of one query head with LSE weights:
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

template <bool F32, int D, bool BATCH>
static void launch_decode_t(int R, int B, int* base, int grid_wg, hipStream_t st,
                            const DecArgs& a) {
  if constexpr (F32) {
    const dim3 grid(a.S, a.Hkv, B);
    switch (R) {
      case 1: hipLaunchKernelGGL((decode_split_kernel<F32, D, 1, BATCH>), grid, dim3(256), 0, st, a); break;
      case 2: hipLaunchKernelGGL((decode_split_kernel<F32, D, 2, BATCH>), grid, dim3(256), 0, st, a); break;
      case 4: hipLaunchKernelGGL((decode_split_kernel<F32, D, 4, BATCH>), grid, dim3(256), 0, st, a); break;
      default: hipLaunchKernelGGL((decode_split_kernel<F32, D, 8, BATCH>), grid, dim3(256), 0, st, a); break;
    }
  } else if constexpr (BATCH) {
    hipLaunchKernelGGL(decode_batch_plan_kernel, dim3(1), dim3(1024), 0, st, a, base, B);
    hipLaunchKernelGGL((decode_mfma_batch_kernel<D>), dim3(grid_wg), dim3(256), 0, st, a,
                       (const int*)base, B);
  } else {
    hipLaunchKernelGGL((decode_mfma_kernel<D>), dim3(a.S * ((a.Hkv + 3) / 4)), dim3(256), 0, st,
                       a);
  }
  hipLaunchKernelGGL((decode_merge_kernel<F32, D, BATCH>), dim3(a.Hq, D / 16, B), dim3(256), 0, st,
                     a);
}

template <bool BATCH>
static void launch_decode_any(int is_f32, int d, int R, int B, int* base, int grid_wg,
                              hipStream_t st, const DecArgs& a) {
  if (is_f32) {
    if (d == 64) launch_decode_t<true, 64, BATCH>(R, B, base, grid_wg, st, a);
    else launch_decode_t<true, 128, BATCH>(R, B, base, grid_wg, st, a);
  } else {
    if (d == 64) launch_decode_t<false, 64, BATCH>(R, B, base, grid_wg, st, a);
    else launch_decode_t<false, 128, BATCH>(R, B, base, grid_wg, st, a);
  }
}

static DecArgs decode_args(const void* xq, const void* kc, const void* vc, void* o, float* lse,
                           int Hq, int Hkv, int64_t w0, float scale, const RopeFreqs& fr,
                           int plain, int cont, void* ws) {
  DecArgs a;
  a.xq = xq;
  a.kc = kc;
  a.vc = vc;
  a.part = (float*)ws;
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
                         void* ws, hipStream_t st) {
  DecArgs a = decode_args(xq, kc, vc, o, lse, Hq, Hkv, w0, scale, fr, plain, cont, ws);
  a.pos = (int)pos;
  a.G = (int)G;
  a.fk_rel = 1.0 / (double)G - 1.0;
  const int keys = (int)pos + 1;
  a.S = (keys + kps - 1) / kps;  // no empty split
  a.kps = kps;
  launch_decode_any<false>(is_f32, d, Hq / Hkv, 1, nullptr, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode_batch(const void* xq, const void* kc, const void* vc, void* o, float* lse,
                               const int32_t* positions, const int32_t* starts, int B,
                               int64_t max_keys, int64_t cap_rows, int Hq, int Hkv, int d,
                               int64_t w0, int64_t w_pre, float scale, const RopeFreqs& fr,
                               int plain, int cont, int is_f32, int splits, int kps, void* ws,
                               int* base, int grid_wg, hipStream_t st) {
  DecArgs a = decode_args(xq, kc, vc, o, lse, Hq, Hkv, w0, scale, fr, plain, cont, ws);
  a.bpos = positions;
  a.bstart = starts;
  a.max_keys = (int)max_keys;
  a.cap_rows = cap_rows;
  a.w_pre = w_pre;
  a.S = splits;
  a.kps = kps;
  launch_decode_any<true>(is_f32, d, Hq / Hkv, B, base, grid_wg, st, a);
  return hipGetLastError();
}

}  // namespace jl
