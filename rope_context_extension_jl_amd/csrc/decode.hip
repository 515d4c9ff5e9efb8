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
// Keys stream in 16-key chunks. A chunk's K and V rows go from HBM straight
// into one of two wave-private LDS stages (direct-to-LDS transfers, no
// registers on the way), so the next chunk is in flight while this one is
// computed. K comes back from LDS as the A operand of S^T = K Q^T (fp16,
// 16x16x32 MFMAs: lane = one key, 8 consecutive dims per 32-dim step); remote
// keys are corrected in-lane, the pairs (i, i + D/2) of a key sitting in
// d-steps ds and ds + D/64 of the same lane. The S^T tile gives each lane one
// query (lane % 16) and four keys, which is the A operand of O = P V in
// 16x16x16 MFMAs; the V operand (4 keys at one dim per lane) comes from the
// transpose read ds_read_b64_tr_b16: within 16 lanes, lane i receives element
// i % 4 of the 8-byte rows addressed by lanes i / 4 + 4t, t = 0..3, so lanes
// pointing at V[key_t][4c .. 4c + 3] deliver V[key_t][own dim] for 4 keys.
// Query heads are padded to the 16 MFMA columns with zeros.
//
// The LDS reads of the stages are inline assembly that waits for its own
// results. Before an LDS read that may touch a transfer's target the compiler
// would wait for every transfer in flight, the next chunk's included; this
// way the only wait on the transfers is the counted one at the top of each
// chunk (transfers complete in issue order).
//
// Softmax: the query operand carries scale * log2(e) and the score
// accumulator starts at -m, m a per-split reference that moves only when a
// lane's sum of bf16-rounded p over the chunk exceeds 2^8 (or on the first
// scores), so the common chunk needs no row max and no cross-lane exchange.
// ---------------------------------------------------------------------------
typedef _Float16 dh8v __attribute__((ext_vector_type(8)));
typedef _Float16 dh2v __attribute__((ext_vector_type(2)));
typedef __bf16 db4v __attribute__((ext_vector_type(4)));
typedef __bf16 db2v __attribute__((ext_vector_type(2)));
typedef short ds4v __attribute__((ext_vector_type(4)));
typedef float df32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t du32x4 __attribute__((ext_vector_type(4)));

constexpr int DEC_CHUNK = 16;  // keys per chunk: one 16-key MFMA block
// chunks per exact (float64) anchor of the correction cos / sin; the others
// take them from the chunk before by one packed fp16 rotation
constexpr int DEC_ANCHOR_CHUNKS = 4;
constexpr float kDecSumMax = 256.f;

template <int D>
struct DecGeom {
  static constexpr int NDS = D / 32;              // 32-dim steps of the QK product
  static constexpr int NDB = D / 16;              // 16-dim output blocks of the PV product
  static constexpr int NC = D / 8;                // 16-byte chunks per key row
  static constexpr int ROW = 2 * D;               // bytes per key row
  static constexpr int RPL = 64 / NC;             // rows per 1 KiB transfer
  static constexpr int XFER = DEC_CHUNK / RPL;    // transfers per array per chunk
  static constexpr int OPS = 2 * XFER;            // transfers per chunk (K and V)
  static constexpr int KBYTES = DEC_CHUNK * ROW;  // K part of a stage, V follows
  static constexpr int STAGE = 2 * KBYTES;        // bytes per LDS stage
};

// LDS slot of 16-byte chunk ch of stage row r: ch ^ dec_swz(r). Rows are 256
// bytes (D = 128), so unswizzled rows would fall on the same banks; with this
// XOR the 16 rows of a K read (the same chunk of every row) hit 16 different
// slots, and the four rows of a V transpose read (a 32-byte chunk pair per
// row) four different pairs.
template <int D>
__device__ __forceinline__ int dec_swz(int r) {
  return ((2 * r) & (DecGeom<D>::NC - 1)) ^ ((r >> 3) & 1);
}

// Per-wave constants of the key loop (all wave-uniform except the lane ids).
struct DecCtx {
  const uint16_t* kbase;  // the head's K row 0
  const uint16_t* vbase;  // the head's V row 0
  int64_t rstride;        // elements between consecutive keys
  int pos, w0, G, plain, correct, k_lo, k_hi;
  int cont;       // remote map x / G (real) instead of floor(x / G)
  double fk_rel;  // with cont: f(k) - k = k * fk_rel
  int lane, g16, r16;
};

template <int D>
struct DecState {
  df32x4 acc[D / 16];  // O: lane holds dims 16 db + r16 of queries 4 g16 + r
  df32x4 negm;         // -m in every element: the QK accumulator's start value
  float m, lsum;       // reference (log2 domain) of query r16, partial row sum
};

// The step from an even chunk's correction cos / sin to the odd chunk's (the
// keys 16 later): f(k + 16) - (k + 16) = f(k) - k + c16 with c16 =
// floor(16 / G) - 16, plus one when (k mod G) + (16 mod G) >= G (floor map;
// never when G divides 16), or exactly 16 / G - 16 (continuous map). c / s
// hold R_{c16}, c1 / s1 R_{c16 + 1}, as fp16 pairs of neighbouring
// frequencies in the key fragments' layout.
template <int D>
struct DecStep {
  dh2v c[D / 64][4], s[D / 64][4];
  dh2v c1[D / 64][4], s1[D / 64][4];
  bool on;       // odd chunks derive their cos / sin from the even ones
  bool carry;    // some keys step by c16 + 1
  int G, r16m;   // G and 16 mod G
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

// Chunk k0's K and V rows -> an LDS stage: transfer i of an array writes rows
// RPL i .. RPL i + RPL - 1 (1 KiB; lane L fills byte 16 L, i.e. row
// RPL i + L / NC, slot L % NC), so lane L fetches that row's chunk
// (L % NC) ^ swz(row). Keys past the split end load the split's last key
// (finite data, masked later), so the loads need no branch.
template <int D>
__device__ __forceinline__ void dec_issue(const DecCtx& c, int k0, uint8_t* stage) {
  using G = DecGeom<D>;
  const int rl = c.lane / G::NC, sl = c.lane % G::NC;
#pragma unroll
  for (int i = 0; i < G::XFER; ++i) {
    const int row = G::RPL * i + rl;
    const int64_t off =
        (int64_t)min(k0 + row, c.k_hi - 1) * c.rstride + 8 * (sl ^ dec_swz<D>(row));
    __builtin_amdgcn_global_load_lds((const void*)(c.kbase + off),
                                     (__attribute__((address_space(3))) void*)(stage + 1024 * i),
                                     16, 0, 2);  // 2: nontemporal
    __builtin_amdgcn_global_load_lds(
        (const void*)(c.vbase + off),
        (__attribute__((address_space(3))) void*)(stage + G::KBYTES + 1024 * i), 16, 0, 2);
  }
}

// The chunk issued before the last one has landed: only the OPS transfers
// of the chunk issued after it may still be in flight.
template <int D>
__device__ __forceinline__ void dec_wait_chunk() {
  static_assert(DecGeom<D>::OPS == 8 || DecGeom<D>::OPS == 4, "transfer count");
  if constexpr (DecGeom<D>::OPS == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
}

// The lane's K fragments of a stage (16 bytes at each of the NDS addresses,
// plus the stage offset OFF); V operands (8 bytes transposed at each of the
// NDB addresses). Each block waits for its own results before it ends, so its
// outputs are complete when the compiler next sees them.
template <int OFF>
__device__ __forceinline__ void dec_read_k(const uint32_t (&a)[4], du32x4 (&k)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%8\n\t"
      "ds_read_b128 %1, %5 offset:%8\n\t"
      "ds_read_b128 %2, %6 offset:%8\n\t"
      "ds_read_b128 %3, %7 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF)
      : "memory");
}
template <int OFF>
__device__ __forceinline__ void dec_read_k(const uint32_t (&a)[2], du32x4 (&k)[2]) {
  asm volatile(
      "ds_read_b128 %0, %2 offset:%4\n\t"
      "ds_read_b128 %1, %3 offset:%4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1])
      : "v"(a[0]), "v"(a[1]), "i"(OFF)
      : "memory");
}
template <int OFF>
__device__ __forceinline__ void dec_read_v(const uint32_t (&a)[8], ds4v (&v)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
      "ds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
      "ds_read_b64_tr_b16 %2, %10 offset:%16\n\t"
      "ds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
      "ds_read_b64_tr_b16 %4, %12 offset:%16\n\t"
      "ds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
      "ds_read_b64_tr_b16 %6, %14 offset:%16\n\t"
      "ds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
        "i"(OFF)
      : "memory");
}
template <int OFF>
__device__ __forceinline__ void dec_read_v(const uint32_t (&a)[4], ds4v (&v)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%8\n\t"
      "ds_read_b64_tr_b16 %1, %5 offset:%8\n\t"
      "ds_read_b64_tr_b16 %2, %6 offset:%8\n\t"
      "ds_read_b64_tr_b16 %3, %7 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF)
      : "memory");
}

// p = exp2(s') of the chunk's 16 keys, packed as the A operand of O = P V;
// returns the lane's sum of the rounded p.
__device__ __forceinline__ float dec_exp(const df32x4& s, ds4v& pb) {
  const db4v p = {(__bf16)__builtin_amdgcn_exp2f(s[0]), (__bf16)__builtin_amdgcn_exp2f(s[1]),
                  (__bf16)__builtin_amdgcn_exp2f(s[2]), (__bf16)__builtin_amdgcn_exp2f(s[3])};
  pb = __builtin_bit_cast(ds4v, p);
  const db2v one = {(__bf16)1.f, (__bf16)1.f};
  const float ps =
      __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), one, 0.f, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), one, ps, false);
}

// One 16-key chunk from LDS stage ST (the even chunks of a split use stage 0,
// the odd ones stage 1). rc / rs carry the even chunk's correction cos / sin
// to the odd one.
template <int D, int ST>
__device__ __forceinline__ void dec_chunk(const DecCtx& c, int k0,
                                          const uint32_t (&ka)[DecGeom<D>::NDS],
                                          const uint32_t (&va)[DecGeom<D>::NDB],
                                          const dh8v (&qa)[D / 32], const dh8v (&qr)[D / 32],
                                          const double (&w2)[D / 64][8], DecState<D>& st,
                                          const DecStep<D>& stp, int kres,
                                          dh2v (&rc)[D / 64][4], dh2v (&rs)[D / 64][4],
                                          float& chk) {
  using G = DecGeom<D>;
  constexpr int NDS = G::NDS, NDB = G::NDB;
  constexpr int KOFF = ST * G::STAGE, VOFF = ST * G::STAGE + G::KBYTES;
  const int key = k0 + c.r16;
  const int klast = min(k0 + DEC_CHUNK - 1, c.k_hi - 1);
  const bool any_rem = !c.plain && c.pos - k0 > c.w0;
  const bool any_loc = c.plain || c.pos - klast <= c.w0;
  const bool fix = c.correct && any_rem;  // the chunk has keys to correct
  // ---- cos / sin of the correction R_{f(k) - k} of the lane's key (pairs
  // (ds, ds + NDS/2), frequencies 32 ds + 8 g16 + j), as fp16 pairs of
  // neighbouring frequencies (j, j + 1), the layout of the key fragments.
  // They depend on the key index only: computed while the chunk's transfers
  // may still be in flight.
  if (fix) {
    if (stp.on && ((k0 - c.k_lo) & (DEC_CHUNK * DEC_ANCHOR_CHUNKS - 1)) != 0) {
      // the chunk k0 - 16 is farther from pos, hence remote too: the
      // rotation moves by the step of the lane's key (kres: the previous
      // key's residue mod G), R_{d + c16} = R_d R_{c16}
      const bool cy = stp.carry && kres + stp.r16m >= stp.G;
#pragma unroll
      for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const dh2v c0 = rc[ds][m], s0 = rs[ds][m];
          const dh2v cs = cy ? stp.c1[ds][m] : stp.c[ds][m];
          const dh2v sn = cy ? stp.s1[ds][m] : stp.s[ds][m];
          rc[ds][m] = c0 * cs - s0 * sn;
          rs[ds][m] = s0 * cs + c0 * sn;
        }
    } else {
      const double delta = c.cont ? (double)key * c.fk_rel : (double)(key / c.G - key);
#pragma unroll
      for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          float c0, s0, c1, s1;
          rope_cs_turns(delta, w2[ds][2 * m], c0, s0);
          rope_cs_turns(delta, w2[ds][2 * m + 1], c1, s1);
          rc[ds][m] = dh2v{(_Float16)c0, (_Float16)c1};
          rs[ds][m] = dh2v{(_Float16)s0, (_Float16)s1};
        }
    }
  }
  dec_wait_chunk<D>();
  // ---- S^T = K Q^T, seeded with -m
  du32x4 kr[NDS];
  dec_read_k<KOFF>(ka, kr);
  dh8v kf[NDS];
  if (fix && c.pos - key > c.w0) {
    // R_{f(k) - k}: absolute -> remapped rotation in packed fp16 arithmetic
    // on two neighbouring frequencies at a time (bf16 keys are exact in fp16)
#pragma unroll
    for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const du32x4 r0 = kr[ds], r1 = kr[ds + NDS / 2];
        const uint32_t w0 = r0[m], w1 = r1[m];
        const dh2v x0 = {(_Float16)__uint_as_float(w0 << 16),
                         (_Float16)__uint_as_float(w0 & 0xffff0000u)};
        const dh2v x1 = {(_Float16)__uint_as_float(w1 << 16),
                         (_Float16)__uint_as_float(w1 & 0xffff0000u)};
        const dh2v y0 = x0 * rc[ds][m] - x1 * rs[ds][m];
        const dh2v y1 = x0 * rs[ds][m] + x1 * rc[ds][m];
        kf[ds][2 * m] = y0[0];
        kf[ds][2 * m + 1] = y0[1];
        kf[ds + NDS / 2][2 * m] = y1[0];
        kf[ds + NDS / 2][2 * m + 1] = y1[1];
      }
  } else {
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) kf[ds] = dec_to_f16(kr[ds]);
  }
  df32x4 s;
  if (!any_loc) {
    dec_qk<D>(kf, qr, st.negm, s);
  } else if (!any_rem) {
    dec_qk<D>(kf, qa, st.negm, s);
  } else {
    // chunk across the window edge: each lane (one key) keeps its fragment
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
    dec_qk<D>(krm, qr, t, s);
  }
  // raw scores of an fp16 operand out of range are not finite: their sum
  // carries that to the end of the split
  chk += (s[0] + s[1]) + (s[2] + s[3]);
  if (klast - k0 < DEC_CHUNK - 1) {  // keys past the split end
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (k0 + 4 * c.g16 + r >= c.k_hi) s[r] = -INFINITY;
  }
  // ---- softmax with the lazy reference
  ds4v pb;
  float psum = dec_exp(s, pb);
  const bool need = !(psum <= kDecSumMax) || st.m == -INFINITY;
  if (__any(need)) {
    // move the reference of the queries that need it to their chunk max; a
    // query's scores live in lanes r16 + 16 g, g = 0..3
    float mt = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
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
    for (int r = 0; r < 4; ++r) s[r] -= delta;
    psum = dec_exp(s, pb);
  }
  st.lsum += psum;
  // ---- O += P V
  ds4v vr[NDB];
  dec_read_v<VOFF>(va, vr);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    st.acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pb, vr[db], st.acc[db], 0, 0, 0);
}

// cos / sin tables a workgroup computes once for the rotations shared by all
// of its lanes: [0][i] of pos * omega_i, [1][i] of f(pos) * omega_i (the
// query at the absolute and the remapped position), [2][i] and [3][i] of
// c16 * omega_i and (c16 + 1) * omega_i (the steps between the two chunks of
// a 32-key pair, see DecStep). One angle per thread.
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
      const double c16 = a.cont ? 16.0 * sq.fk_rel : (double)(16 / sq.G - 16);
      rope_cs_turns(c16, w, c, s);
      tab[2][i] = make_float2(c, s);
      rope_cs_turns(c16 + 1.0, w, c, s);
      tab[3][i] = make_float2(c, s);
    }
  }
}

// Whether the odd chunk of a 32-key pair takes its cos / sin from the even
// one by one rotation (see DecStep): whenever keys are corrected.
__device__ __forceinline__ bool dec_step16(const DecArgs& a, const DecSeq& sq) {
  return !a.plain && sq.G > 1;
}

// Workgroup barrier for the LDS tables: every ds_read / ds_write issued
// before it has completed, and the compiler moves no memory access across
// it. Global loads and the transfers into the waves' private stages stay in
// flight (__syncthreads, and any LDS fence, would wait for all of them: a
// transfer's LDS write is counted with the vector memory operations).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Per-wave constants of one work unit: keys [s kps, (s + 1) kps) of KV head
// kvh of sequence sq.
template <int D>
__device__ __forceinline__ DecCtx dec_ctx(const DecArgs& a, const DecSeq& sq, int s, int kvh) {
  const int lane = threadIdx.x & 63;
  DecCtx c;
  c.k_lo = s * a.kps;
  c.k_hi = min(c.k_lo + a.kps, sq.pos + 1);
  c.rstride = (int64_t)a.Hkv * D;
  c.kbase = (const uint16_t*)sq.kc + (int64_t)kvh * D;
  c.vbase = (const uint16_t*)sq.vc + (int64_t)kvh * D;
  c.pos = sq.pos;
  c.w0 = a.w0;
  c.G = sq.G;
  c.cont = a.cont;
  c.fk_rel = sq.fk_rel;
  c.plain = a.plain;
  c.correct = !a.plain && sq.G > 1;
  c.lane = lane;
  c.g16 = lane >> 4;
  c.r16 = lane & 15;
  return c;
}

// The lane's raw query elements: dims 32 ds + 8 g16 .. + 8 (lo) and their
// partners + D/2 (hi) of query head r16 of the group, as 16-byte loads of a
// valid row (head r16 clamped; the rotation zeroes heads past the group).
template <int D>
struct DecQRaw {
  du32x4 lo[D / 64], hi[D / 64];
};

// Start of a work unit, before the rotation tables exist: the raw query
// loads and the transfers of the first chunk (stage 0) go out, so the first
// round trip to memory overlaps the table set-up.
template <int D>
__device__ __forceinline__ void dec_begin(const DecArgs& a, const DecSeq& sq, int kvh,
                                          const DecCtx& c, DecQRaw<D>& raw, uint8_t* stages) {
  const int R = a.Hq / a.Hkv;
  const uint16_t* qp = (const uint16_t*)sq.xq + (int64_t)(kvh * R + (c.r16 < R ? c.r16 : 0)) * D;
#pragma unroll
  for (int ds = 0; ds < D / 64; ++ds) {
    raw.lo[ds] = *(const du32x4*)(qp + 32 * ds + 8 * c.g16);
    raw.hi[ds] = *(const du32x4*)(qp + 32 * ds + 8 * c.g16 + D / 2);
  }
  __builtin_amdgcn_sched_barrier(0);
  dec_issue<D>(c, c.k_lo, stages);
  __builtin_amdgcn_sched_barrier(0);
}

// One work unit of the bf16 decode for one wave, after dec_begin: keys
// [c.k_lo, c.k_hi) of KV head kvh of sequence sq, leaving the partial of each
// query head of the group. stages: this wave's two LDS stages (2 * STAGE
// bytes), the first holding (in flight) the unit's first chunk.
template <int D>
__device__ __forceinline__ void dec_unit(const DecArgs& a, const DecSeq& sq, int s, int kvh,
                                         const DecCtx& c, const DecQRaw<D>& raw,
                                         const double* w2pi_s, const float2 (*tab)[D / 2],
                                         uint8_t* stages) {
  using G = DecGeom<D>;
  constexpr int NDS = G::NDS, NDB = G::NDB;
  const int g16 = c.g16, r16 = c.r16;
  const int R = a.Hq / a.Hkv, h0 = kvh * R;
  const int k_lo = c.k_lo;

  // LDS addresses of the lane's reads, relative to a stage's K or V part
  // (the stage and part offsets are immediates of the reads): K row r16,
  // chunks 4 ds + g16 (dims 32 ds + 8 g16 .. + 8); for the V transpose reads
  // row 4 g16 + r16 / 4, dims 16 db + 4 (r16 % 4) .. + 3, i.e. byte
  // 8 (r16 & 1) of chunk 2 db + (r16 & 3) / 2
  uint32_t ka[NDS], va[NDB];
  {
    const uint32_t sb =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)stages;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      ka[ds] = sb + r16 * G::ROW + 16 * ((4 * ds + g16) ^ dec_swz<D>(r16));
    const int vrow = 4 * g16 + (r16 >> 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      va[db] = sb + vrow * G::ROW +
               16 * ((2 * db + ((r16 & 3) >> 1)) ^ dec_swz<D>(vrow)) + 8 * (r16 & 1);
  }

  // query operands (B of S^T = K Q^T): lane holds dims 32 ds + 8 g16 + j of
  // query head r16, rotated at pos (qa) and at f(pos) (qr), times scale*log2 e
  dh8v qa[NDS], qr[NDS];
  {
    const bool qv = r16 < R;
#pragma unroll
    for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 32 * ds + 8 * g16 + j;
        const float x0 = qv ? bf16_lane(raw.lo[ds], j) : 0.f;
        const float x1 = qv ? bf16_lane(raw.hi[ds], j) : 0.f;
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
  // the lane's correction frequencies (in turns), held in registers: the key
  // loop reads no LDS outside its stages
  double w2[NDS / 2][8];
#pragma unroll
  for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
    for (int j = 0; j < 8; ++j) w2[ds][j] = w2pi_s[32 * ds + 8 * g16 + j];
  // the steps between the two chunks of a pair (see DecStep)
  DecStep<D> stp;
  stp.on = dec_step16(a, sq);
  stp.carry = stp.on && !a.cont && 16 % sq.G != 0;
  stp.G = sq.G;
  stp.r16m = 16 % sq.G;
  if (stp.on) {
#pragma unroll
    for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int i = 32 * ds + 8 * g16 + 2 * m;
        float2 t0 = tab[2][i], t1 = tab[2][i + 1];
        stp.c[ds][m] = dh2v{(_Float16)t0.x, (_Float16)t1.x};
        stp.s[ds][m] = dh2v{(_Float16)t0.y, (_Float16)t1.y};
        t0 = tab[3][i];
        t1 = tab[3][i + 1];
        stp.c1[ds][m] = dh2v{(_Float16)t0.x, (_Float16)t1.x};
        stp.s1[ds][m] = dh2v{(_Float16)t0.y, (_Float16)t1.y};
      }
  }
  // residue mod G of the lane's key in the even chunk of the current pair;
  // pairs advance by 32 keys
  // residue mod G of the lane's key in the chunk before the one computed
  int kres = ((k_lo + r16) % sq.G + sq.G - stp.r16m) % sq.G;
  auto advance = [&]() { kres = kres + stp.r16m >= sq.G ? kres + stp.r16m - sq.G : kres + stp.r16m; };

  DecState<D> st;
#pragma unroll
  for (int db = 0; db < NDB; ++db) st.acc[db] = df32x4{0.f, 0.f, 0.f, 0.f};
  st.negm = df32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.lsum = 0.f;
  float chk = 0.f;
  dh2v rc[NDS / 2][4], rs[NDS / 2][4];

  // chunk i + 1 is in flight while chunk i is computed; the next chunk is
  // always issued (past the split end it re-reads the last key, from L2).
  // Chunks alternate between the two stages; a stage is refilled only after
  // the chunk that read it, whose reads have completed.
  for (int k0 = k_lo;; k0 += 2 * DEC_CHUNK) {
    dec_issue<D>(c, k0 + DEC_CHUNK, stages + G::STAGE);
    __builtin_amdgcn_sched_barrier(0);  // the transfers go out first
    dec_chunk<D, 0>(c, k0, ka, va, qa, qr, w2, st, stp, kres, rc, rs, chk);
    advance();
    if (k0 + DEC_CHUNK >= c.k_hi) break;
    dec_issue<D>(c, k0 + 2 * DEC_CHUNK, stages);
    __builtin_amdgcn_sched_barrier(0);
    dec_chunk<D, 1>(c, k0 + DEC_CHUNK, ka, va, qa, qr, w2, st, stp, kres, rc, rs, chk);
    advance();
    if (k0 + 2 * DEC_CHUNK >= c.k_hi) break;
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
  __shared__ __attribute__((aligned(16))) uint8_t stg[4][2 * G::STAGE];  // two stages per wave
  __shared__ double w2pi_s[D / 2];
  __shared__ float2 tab_s[4][D / 2];
  // the wave index is uniform per wave: say so, so that every split-derived
  // value (key range, route of a key block) lives in scalar registers and the
  // route branches are scalar jumps; matrix instructions then never run under
  // a partial or empty EXEC mask
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const DecSeq sq = dec_seq<false>(a, 0, D, 2);
  const int hgroups = (a.Hkv + 3) >> 2;
  const int s = blockIdx.x / hgroups, kvh = (blockIdx.x % hgroups) * 4 + wave;
  // a wave past the last KV head starts the last head's unit too (in-bounds
  // reads, no branch around the transfers) and drops it after the tables
  const bool live = kvh < a.Hkv;
  const int kvu = live ? kvh : a.Hkv - 1;
  const DecCtx c = dec_ctx<D>(a, sq, s, kvu);
  DecQRaw<D> raw;
  dec_begin<D>(a, sq, kvu, c, raw, stg[wave]);
  if (tid < D / 2) w2pi_s[tid] = a.fr.w(tid) * kInvTwoPi;
  lds_barrier();
  dec_tables<D>(a, sq, dec_step16(a, sq), w2pi_s, tab_s);
  lds_barrier();
  if (!live) {
    __builtin_amdgcn_s_waitcnt(0);  // no transfer outlives the wave
    return;
  }
  dec_unit<D>(a, sq, s, kvh, c, raw, w2pi_s, tab_s, stg[wave]);
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
  __shared__ __attribute__((aligned(16))) uint8_t stg[4][2 * G::STAGE];  // two stages per wave
  __shared__ double w2pi_s[D / 2];
  __shared__ float2 tab_s[4][D / 2];
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
    // this wave's stages are free: its previous unit waited for them; a wave
    // past the last KV head starts the last head's unit and drops it
    const bool live = kvh < a.Hkv;
    const int kvu = live ? kvh : a.Hkv - 1;
    const int s = item - base[lo];
    const DecCtx c = dec_ctx<D>(a, sq, s, kvu);
    DecQRaw<D> raw;
    dec_begin<D>(a, sq, kvu, c, raw, stg[wave]);
    // this unit's tables (every wave passes both barriers, also the waves
    // past the last KV head)
    lds_barrier();
    dec_tables<D>(a, sq, dec_step16(a, sq), w2pi_s, tab_s);
    lds_barrier();
    if (!live) {
      __builtin_amdgcn_s_waitcnt(0);  // the stages are free for the next unit
      continue;
    }
    dec_unit<D>(a, sq, s, kvh, c, raw, w2pi_s, tab_s, stg[wave]);
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
