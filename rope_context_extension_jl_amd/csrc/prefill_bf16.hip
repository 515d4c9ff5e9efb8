// Bifocal prefill for bf16 I/O on gfx950: plan, key/value pre-pass, fused
// MFMA attention pass, device tile-class dump.
//
// Method (r9-hu digest of Jet-Long, section Method): Eq. 1 routes each
// query/key pair by distance -- q - k <= w0 scores the vectors rotated at
// (q, k), otherwise at (f(q), f(k)) with f(x) = floor(x / G) and
// G = max(1, ceil(L / w_pretrained)) per sequence ("Dynamic group size").
//
// Design:
//   * The pre-pass rotates every raw key ONCE to its absolute and its
//     remapped position (fp32 arithmetic, float64-reduced angles) and stores
//     both as fp16 tiles in the workspace, head-major and padded so every
//     sequence starts on a 64-row boundary. It also writes V transposed
//     (d-major, each 16-key group in the PV operand's key order) so the PV
//     product reads 16-byte MFMA operands, and optionally the bf16 absolute
//     key cache.
//   * The attention kernel gives each workgroup (4 waves, 256 threads) 128
//     query rows of one query head. Each lane of a wave owns ONE query row:
//     scores are computed transposed, S^T = K Q^T, so the 32x32 MFMA output
//     puts a row's scores in one lane (plus its partner lane l^32) and the
//     row max / row sum need a single cross-lane exchange.
//   * Every 64-key tile is classified (local / remote / boundary, plus the
//     causal diagonal) from distances only. Local tiles use the absolute
//     operands, remote tiles the remapped ones, boundary tiles compute both
//     products and select per element; only boundary tiles (a few tenths of
//     a percent at 64K-128K) pay for the second product.
//   * QK^T uses fp16 operands (the rotated vectors keep the raw norm, so the
//     fp16 range holds them, and fp16 carries 3 more mantissa bits than bf16
//     at the same MFMA rate); PV uses bf16 P and the raw bf16 V. Accumulation
//     is fp32 throughout; O is rounded to bf16 once.
//   * When Hq / Hkv is even, every pass (fused, plain, the three of Eq. 7)
//     runs two query heads of one KV head per workgroup (8 waves, one
//     workgroup per CU) over a 3-stage LDS pipeline; the 4-wave kernel, one
//     head per workgroup, serves odd ratios.
//   * The schedule hands the heaviest query tiles out first (longest causal
//     key range), and consecutive workgroups of one XCD share a KV head so
//     the key tiles they stream stay in that XCD's L2.
#include "jl_internal.hpp"

namespace jl {

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef __bf16 b8v __attribute__((ext_vector_type(8)));
typedef __bf16 b2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// native 16-byte vector (HIP's uint4 is a struct with a union, which keeps
// arrays of it out of registers)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// LDS stages are filled by direct global -> LDS transfers (16 bytes per lane,
// placed contiguously), so rows are not padded; instead the 16-byte chunks of
// a row are XOR-swizzled by the row: a key row (128 fp16 = 256 B, 16 chunks)
// by row & 15, a value^T row (64 bf16 = 128 B, 8 chunks) by (row >> 1) & 7.
// The 16 lanes reading one operand chunk then hit 16 distinct bank groups.
__device__ __forceinline__ int kswz(int row) { return row & 15; }
__device__ __forceinline__ int vswz(int row) { return (row >> 1) & 7; }

// Position q (0..15) of a 16-key group in the value^T layout (workspace and
// LDS) holds key vperm(q) of the group: keys {0-3, 8-11, 4-7, 12-15}, so the
// 8 keys of a lane's PV operand (see softmax_pv_any) are one 16-byte chunk.
__device__ __forceinline__ int vperm(int q) {
  return (((q >> 2) ^ (q >> 3)) & 1) ? q ^ 12 : q;
}

// ---------------------------------------------------------------------------
// Plan: per-sequence records and the heaviest-first tile order.
//   seqs[b]   = {start, len, G, pad_off}
//   order[rho]: sequences sorted by query-tile count, descending (ties by b)
//   tact[t]   = number of sequences with more than t query tiles
//   tbase[t]  = sum of tact[t'] over t' > t
// Slot s of the schedule is tile depth t (smallest t with tbase[t] <= s) of
// sequence order[s - tbase[t]]: deepest (heaviest) tiles first.
// hdr[0] = number of tiles, hdr[1] = deepest tile count, hdr[2] = padded rows,
// hdr[3] = range flags of this call (cleared here, OR-ed by the later kernels).
// ---------------------------------------------------------------------------
constexpr int PLAN_THREADS = 1024;

__device__ inline int block_excl_scan(int v, int* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < PLAN_THREADS; off <<= 1) {
    int add = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  int incl = sh[tid];
  int total = sh[PLAN_THREADS - 1];
  __syncthreads();
  sh[PLAN_THREADS] = total;
  return incl - v;
}

__global__ void __launch_bounds__(PLAN_THREADS) prefill_plan_kernel(
    const int32_t* __restrict__ cu, int B, int T, int qoff, int64_t w_pre, int bm,
    int* __restrict__ hdr,
    SeqInfo* __restrict__ seqs, int* __restrict__ order, int* __restrict__ tact,
    int* __restrict__ tbase) {
  // Every value one thread produces for another goes through LDS (B <= 4096).
  __shared__ int nt_s[4096];
  __shared__ int len_s[4096];
  __shared__ int ord_s[4096];
  __shared__ int sh[PLAN_THREADS + 1];
  __shared__ int maxnt_s;
  const int tid = threadIdx.x;
  if (tid == 0) {
    maxnt_s = 0;
    hdr[kHdrFlags] = 0;
  }
  __syncthreads();
  for (int b = tid; b < B; b += PLAN_THREADS) {
    const int s = cu ? cu[b] : 0;
    const int e = cu ? cu[b + 1] : T;
    const int len = e > s ? e - s : 0;
    len_s[b] = len;
    // query tiles: the rows from qoff on (qoff > 0 only for one sequence
    // continued on an existing cache: its first qoff rows are keys only)
    nt_s[b] = (len - qoff + bm - 1) / bm;
    atomicMax(&maxnt_s, nt_s[b]);
    seqs[b].start = s;
    seqs[b].len = len;
    seqs[b].G = (int)group_size(len > 0 ? len : 1, w_pre);
  }
  __syncthreads();
  // pad_off: exclusive prefix sum of the 64-rounded lengths, `per` per thread
  {
    const int per = (B + PLAN_THREADS - 1) / PLAN_THREADS;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int b = tid * per + i;
      if (b < B) local += (len_s[b] + 63) & ~63;
    }
    int run = block_excl_scan(local, sh);
    if (tid == 0) hdr[2] = sh[PLAN_THREADS];
    for (int i = 0; i < per; ++i) {
      const int b = tid * per + i;
      if (b < B) {
        seqs[b].pad_off = run;
        run += (len_s[b] + 63) & ~63;
      }
    }
  }
  // stable rank by tile count, descending
  for (int b = tid; b < B; b += PLAN_THREADS) {
    int rank = 0;
    const int nb = nt_s[b];
    for (int c = 0; c < B; ++c) rank += (nt_s[c] > nb) || (nt_s[c] == nb && c < b);
    ord_s[rank] = b;
  }
  __syncthreads();
  for (int i = tid; i < B; i += PLAN_THREADS) order[i] = ord_s[i];
  const int maxnt = maxnt_s;
  // tact[t] = #{rho : nt[order[rho]] > t} (sorted counts are non-increasing);
  // tbase[t] = sum of tact[t'] over t' > t, scanned in order of decreasing t.
  int carry = 0;
  for (int c0 = 0; c0 < maxnt; c0 += PLAN_THREADS) {
    const int u = c0 + tid;
    const int t = maxnt - 1 - u;
    int act = 0;
    if (u < maxnt) {
      int lo = 0, hi = B;  // first rho with nt <= t
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (nt_s[ord_s[mid]] > t) lo = mid + 1; else hi = mid;
      }
      act = lo;
    }
    const int ex = block_excl_scan(act, sh);
    if (u < maxnt) {
      tact[t] = act;
      tbase[t] = carry + ex;
    }
    carry += sh[PLAN_THREADS];
    __syncthreads();
  }
  if (tid == 0) {
    hdr[0] = carry;  // total tiles
    hdr[1] = maxnt;
  }
}

hipError_t launch_prefill_plan(const int32_t* cu, int B, int64_t T, int64_t qoff, int64_t w_pre,
                               int bm, void* ws, const PrefillLayout& lay, hipStream_t st) {
  char* w = (char*)ws;
  int* order = (int*)(w + lay.tiles);
  int* tact = order + B;
  int* tbase = tact + (lay.max_tiles + 1);
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, st, cu, B, (int)T,
                     (int)qoff, w_pre, bm, (int*)(w + lay.hdr), (SeqInfo*)(w + lay.seqs), order, tact, tbase);
  return hipGetLastError();
}

__device__ inline int seq_of_padded_row(const SeqInfo* seqs, int B, int r) {
  int lo = 0, hi = B - 1;  // largest b with pad_off <= r
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (seqs[mid].pad_off <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// Pre-pass: 64 padded rows per workgroup (rows of one sequence, or padding).
// With from_abs the keys are already rotated at their absolute positions (an
// existing key cache): the absolute operand is the key itself and the
// remapped one is R_{f(k) - k} applied to it (R_a R_b = R_{a+b}).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) prefill_prep_bf16_kernel(
    const uint16_t* __restrict__ xk, const uint16_t* __restrict__ v, uint16_t* __restrict__ kcache,
    const SeqInfo* __restrict__ seqs, const int* __restrict__ hdr, int B, int Hkv, int R,
    int need_rem, int from_abs, float kscale, int cont, uint16_t* __restrict__ kabs,
    uint16_t* __restrict__ krem, uint16_t* __restrict__ vt, RopeFreqs fr, int* __restrict__ flags) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * (PF_D + 8)];
  const int r0 = blockIdx.x * 64;
  if (r0 >= hdr[2]) return;
  uint32_t nonfinite = 0;  // OR of (fp16 bits & 0x7c00) == 0x7c00 over the key operands
  const int b = seq_of_padded_row(seqs, B, r0);
  const SeqInfo sq = seqs[b];
  const int tid = threadIdx.x;
  // keys: thread = (row, pair group of 8); two passes of 32 rows
  for (int pass = 0; pass < 2; ++pass) {
    const int i = pass * 32 + (tid >> 3);
    const int c = tid & 7;
    const int r = r0 + i;
    const int trel = r - sq.pad_off;
    const bool valid = trel < sq.len;
    float ca[8], sa[8], cr[8], sr[8];
    const double pa = from_abs ? 0.0 : (double)trel;
    const double fk = remap_pos(trel, sq.G, cont);
    const double pr = from_abs ? fk - (double)trel : fk;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      rope_cs(pa, fr.w(8 * c + j), ca[j], sa[j]);
      if (need_rem) rope_cs(pr, fr.w(8 * c + j), cr[j], sr[j]);
    }
    for (int g = 0; g < Hkv; ++g) {
      uint4 av = make_uint4(0, 0, 0, 0), bv = av;
      if (valid) {
        const uint16_t* src = xk + ((int64_t)(sq.start + trel) * Hkv + g) * PF_D;
        av = *(const uint4*)(src + 8 * c);
        bv = *(const uint4*)(src + 64 + 8 * c);
      }
      const uint16_t* ap = (const uint16_t*)&av;
      const uint16_t* bp = (const uint16_t*)&bv;
      uint16_t oa[8], ob[8], ra[8], rb[8], ka[8], kb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x0 = bf16_bits_to_f32(ap[j]), x1 = bf16_bits_to_f32(bp[j]);
        const float y0 = x0 * ca[j] - x1 * sa[j], y1 = x0 * sa[j] + x1 * ca[j];
        oa[j] = f32_to_f16_bits(y0 * kscale);
        ob[j] = f32_to_f16_bits(y1 * kscale);
        ka[j] = f32_to_bf16_bits(y0);
        kb[j] = f32_to_bf16_bits(y1);
        if (need_rem) {
          ra[j] = f32_to_f16_bits((x0 * cr[j] - x1 * sr[j]) * kscale);
          rb[j] = f32_to_f16_bits((x0 * sr[j] + x1 * cr[j]) * kscale);
          nonfinite |= f16_nonfinite(ra[j]) | f16_nonfinite(rb[j]);
        }
        nonfinite |= f16_nonfinite(oa[j]) | f16_nonfinite(ob[j]);
      }
      uint16_t* da = kabs + ((int64_t)g * R + r) * PF_D;
      *(uint4*)(da + 8 * c) = *(const uint4*)oa;
      *(uint4*)(da + 64 + 8 * c) = *(const uint4*)ob;
      if (need_rem) {
        uint16_t* dr = krem + ((int64_t)g * R + r) * PF_D;
        *(uint4*)(dr + 8 * c) = *(const uint4*)ra;
        *(uint4*)(dr + 64 + 8 * c) = *(const uint4*)rb;
      }
      if (kcache && valid) {
        uint16_t* dc = kcache + ((int64_t)(sq.start + trel) * Hkv + g) * PF_D;
        *(uint4*)(dc + 8 * c) = *(const uint4*)ka;
        *(uint4*)(dc + 64 + 8 * c) = *(const uint4*)kb;
      }
    }
  }
  if (nonfinite) atomicOr(flags, JL_FLAG_K_RANGE);
  // values: transpose 64 rows x 128 per KV head through LDS
  for (int g = 0; g < Hkv; ++g) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = (tid >> 4) + 16 * k, c = tid & 15;
      const int trel = r0 + i - sq.pad_off;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (trel < sq.len) val = *(const uint4*)(v + ((int64_t)(sq.start + trel) * Hkv + g) * PF_D + 8 * c);
      *(uint4*)(tile + i * (PF_D + 8) + 8 * c) = val;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int dd = (tid >> 3) + 32 * k, kc = tid & 7;
      uint16_t out[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int pos = 8 * kc + e;  // column of the 64-key row, in the vperm order
        out[e] = tile[(16 * (pos >> 4) + vperm(pos & 15)) * (PF_D + 8) + dd];
      }
      *(uint4*)(vt + ((int64_t)g * PF_D + dd) * R + r0 + 8 * kc) = *(const uint4*)out;
    }
    __syncthreads();
  }
}

hipError_t launch_prefill_prep_bf16(const void* xk, const void* v, void* kcache_out, int64_t T,
                                    int B, int Hkv, int need_rem, int from_abs, float kscale,
                                    int cont, const RopeFreqs& fr, void* ws,
                                    const PrefillLayout& lay, hipStream_t st) {
  char* w = (char*)ws;
  const int blocks = (int)(lay.R / 64);
  hipLaunchKernelGGL(prefill_prep_bf16_kernel, dim3(blocks), dim3(256), 0, st,
                     (const uint16_t*)xk, (const uint16_t*)v, (uint16_t*)kcache_out,
                     (const SeqInfo*)(w + lay.seqs), (const int*)(w + lay.hdr), B, Hkv,
                     (int)lay.R, need_rem, from_abs, kscale, cont, (uint16_t*)(w + lay.kabs),
                     (uint16_t*)(w + lay.krem), (uint16_t*)(w + lay.vt), fr,
                     (int*)(w + lay.hdr) + kHdrFlags);
  (void)T;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Attention pass.
// ---------------------------------------------------------------------------
struct PfArgs {
  const uint16_t* xq;    // raw bf16 [T, Hq, D]
  const uint16_t* kabs;  // fp16 [Hkv, R, D]
  const uint16_t* krem;  // fp16 [Hkv, R, D]
  const uint16_t* vt;    // bf16 [Hkv, D, R]
  void* o;               // bf16 [T, Hq, D] (fp32 for the inclusion-exclusion passes)
  float* lse;            // [Hq, T] or null
  const SeqInfo* seqs;
  const int* hdr;
  const int* order;
  const int* tact;
  const int* tbase;
  int T, R, Hq, Hkv, w0;
  int qoff;       // position of the first query row (0 unless continuing on a cache)
  int ie_remote;  // pass B of Eq. 7 (1) or pass C (0)
  int cont;       // remote map x / G (real) instead of floor(x / G)
  RopeFreqs fr;
  int* flags;     // range flags word of the workspace header
};

__device__ inline float xor32(float x) { return __shfl_xor(x, 32); }

enum MaskMode : int { MASK_NONE = 0, MASK_WINDOW = 1, MASK_REMOTE = 2 };

// Per-workgroup constants of the attention pass. Everything the key loop
// needs is copied here from the kernel arguments so that no pointer to the
// argument block is taken (which would force it, and every pointer loaded
// from it, into generic/private memory).
struct Tctx {
  const uint16_t* kabs;  // this sequence's KV head, row 0 of the padded layout
  const uint16_t* krem;
  const uint16_t* vt;    // column 0 of the sequence in the transposed values
  int R;                 // padded row stride of vt
  int q0, q1, len, nkt, w0;
  int tid, hh, l32, myq;
  // this lane's first source byte of its tile transfers (tile 0), fixed for
  // the whole walk, and the byte step between a lane's value transfers: the
  // per-tile address is then one uniform offset away
  const char* kabs_l;
  const char* krem_l;
  const char* vt_l;
  int64_t vstep;
};

// Running softmax state of one lane's query row. Scores come out of the
// MFMA in the log2 domain, already shifted by the reference: the key
// operands carry c = scale * log2(e) (applied in the pre-pass before their
// fp16 rounding) and the QK^T accumulator starts at -m, so each output is
// s' = c (q . k) - m and p = exp2(s'). The query operand is the rotated query
// itself.
struct RowState {
  f32x16 acc[4];  // O^T accumulator: d = 32*db + 8*(r/4) + 4*hh + r%4
  f32x16 negm;    // -m in every register: the QK^T accumulator's start value
  float m, l;     // reference (log2 domain; -inf until the row has a score)
                  // and this lane's partial sum
};

__device__ __forceinline__ int tile_cls_of(const Tctx& c, int j) {
  const int k0 = j * PF_BN;
  return tile_class(c.q0, c.q1, k0, min(k0 + PF_BN, c.len) - 1, c.w0);
}

// Global -> LDS stage of key tile j (64 x 128 fp16, remapped or absolute) and
// value^T tile j (128 x 64 bf16) by direct transfers, no registers: 16
// transfers of 1 KiB each per tile, transfer o = w + 4 i issued by wave w.
// Lane L of a transfer fills the 16 bytes at 16 L of its window, i.e. row
// (window start) + L / 16 (keys) or + L / 8 (values) at physical chunk L % 16
// (L % 8), and fetches the logical chunk the swizzle puts there. With this
// interleaving a lane's swizzle is the same in all four of its transfers,
// so its source address advances by a constant per transfer.
__device__ __forceinline__ void tile_dma(const Tctx& c, int j, bool rem, uint16_t* ks,
                                         uint16_t* vs) {
  const int w = __builtin_amdgcn_readfirstlane(c.tid >> 6);
  const char* kg = (rem ? c.krem_l : c.kabs_l) + (int64_t)j * (PF_BN * PF_D * 2);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_global_load_lds(
        (const void*)(kg + 16 * PF_D * 2 * i),
        (__attribute__((address_space(3))) void*)(ks + 512 * (w + 4 * i)), 16, 0, 0);
  const char* vg = c.vt_l + (int64_t)j * (PF_BN * 2);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_global_load_lds(
        (const void*)(vg + c.vstep * i),
        (__attribute__((address_space(3))) void*)(vs + 512 * (w + 4 * i)), 16, 0, 0);
}
// The lane's tile-0 sources of tile_dma (NW = 4) or tile_dma8 (NW = 8): key
// row 4 w + L / 16 of the tile at swizzled chunk (L % 16) ^ kswz(row);
// value^T row 8 w + L / 8 at chunk (L % 8) ^ vswz(row); a value transfer
// moves on by 8 NW rows.
template <int NW>
__device__ __forceinline__ void tile_dma_lanes(Tctx& c) {
  const int w = __builtin_amdgcn_readfirstlane(c.tid >> 6), lane = c.tid & 63;
  const int rk = 4 * w + (lane >> 4), lk = (lane & 15) ^ kswz(rk);
  const int rv = 8 * w + (lane >> 3), lv = (lane & 7) ^ vswz(rv);
  c.kabs_l = (const char*)(c.kabs + rk * PF_D + 8 * lk);
  c.krem_l = (const char*)(c.krem + rk * PF_D + 8 * lk);
  c.vt_l = (const char*)(c.vt + (int64_t)rv * c.R + 8 * lv);
  c.vstep = (int64_t)(8 * NW) * c.R * 2;
}
// End of a tile: this wave's transfers into the other stage have landed,
// then every wave is past its reads of this stage.
__device__ __forceinline__ void tile_sync() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// The two LDS stages (key, value^T) x 2; the stage a tile uses is picked at
// run time. Reads of a stage and the transfers in flight into the other
// touch disjoint LDS; the wait + barrier at the end of each tile orders a
// transfer before the reads of its data.
struct Stages {
  uint16_t *k0, *v0, *k1, *v1;
};

// S^T (two 32-key blocks) = K Q^T for the key tile in LDS. The A operand is a
// key row slice d = 16c + 8hh .. +8, the B operand the same slice of the
// lane's query row; the MFMA's k-index mapping is the same for both.
__device__ __forceinline__ void qk_lds(const Tctx& c, const uint16_t* ks, const h8v (&q)[8],
                                       const f32x16& negm, f32x16 (&s)[2]) {
  const int x = kswz(c.l32);
#pragma unroll
  for (int bk = 0; bk < 2; ++bk) {
    const uint16_t* krow = ks + (32 * bk + c.l32) * PF_D;
    s[bk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const h8v*)(krow + 8 * (c.hh ^ x)), q[0],
                                                   negm, 0, 0, 0);
#pragma unroll
    for (int cc = 1; cc < 8; ++cc)
      s[bk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
          *(const h8v*)(krow + 8 * ((2 * cc + c.hh) ^ x)), q[cc], s[bk], 0, 0, 0);
  }
}

// Boundary tile of the fused pass: remapped scores from the global key tile,
// element-wise select by the route of Eq. 1.
__device__ __forceinline__ void boundary_select(const Tctx& c, int j, const h8v (&qr)[8],
                                                const f32x16& negm, f32x16 (&s)[2]) {
  const int k0 = j * PF_BN;
#pragma unroll
  for (int bk = 0; bk < 2; ++bk) {
    const uint16_t* krow = c.krem + (int64_t)(k0 + 32 * bk + c.l32) * PF_D + 8 * c.hh;
    f32x16 s2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const h8v*)krow, qr[0], negm, 0, 0, 0);
#pragma unroll
    for (int cc = 1; cc < 8; ++cc)
      s2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const h8v*)(krow + 16 * cc), qr[cc], s2, 0, 0,
                                                  0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = k0 + 32 * bk + 8 * (r >> 2) + 4 * c.hh + (r & 3);
      if (c.myq - kk > c.w0) s[bk][r] = s2[r];
    }
  }
}

// Masks, online softmax and O^T += V^T P^T for one tile whose shifted
// scores s' = c (q . k) - m are in s. The reference m does not follow every new
// row maximum: it moves only when the tile's probabilities p = exp2(s') summed
// over a lane's 32 keys exceed 2^64 (or the row has no reference yet), so
// every p stays below 2^64 and the sum check replaces the per-tile row max.
// Since the final division uses the same reference, the result does not
// depend on where the reference sits (p is rounded to bf16 with the same
// relative error at any magnitude); the rescale of the 64 accumulator
// registers, the row max and the cross-lane exchange are skipped on almost
// every tile. The tile sum is taken over the bf16-rounded p, the same values
// the PV product weights, so numerator and denominator see identical p.
// Bound: a row's l and |acc| stay below 2^65 per key tile times max |v| (at
// 2048 key tiles, finite for |v| < 2^50). A small bound moves the reference
// whenever some row's maximum grows by its log2; rows scored against a few
// large keys then move it tens of times per walk (2^8: 53-58 moves per wave
// over a 2048-tile walk at 128K, 2^64: the first tile only, simulated), each
// on the rarely taken branch that every other wave waits for at the tile
// barrier.
constexpr float kSumMax = 0x1p64f;

// Causal / window masks on the raw scores of a tile that needs them.
__device__ __forceinline__ void mask_scores(const Tctx& c, int j, int cls, int mask_mode,
                                            f32x16 (&s)[2]) {
  const int k0 = j * PF_BN;
  const bool causal = (cls & TC_DIAG) || j == c.nkt - 1;
  const bool bnd = (cls & 3) == TC_BOUNDARY;
  const bool window = bnd && mask_mode == MASK_WINDOW;       // keep q - k <= w0
  const bool remote_only = bnd && mask_mode == MASK_REMOTE;  // keep q - k >  w0
#pragma unroll
  for (int bk = 0; bk < 2; ++bk)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = k0 + 32 * bk + 8 * (r >> 2) + 4 * c.hh + (r & 3);
      const int dist = c.myq - kk;
      const bool drop = (causal && dist < 0) || (window && dist > c.w0) ||
                        (remote_only && dist <= c.w0);
      if (drop) s[bk][r] = -INFINITY;
    }
}

// Does tile j need masks?
__device__ __forceinline__ bool tile_needs_mask(const Tctx& c, int j, int cls, int mask_mode) {
  return (cls & TC_DIAG) || j == c.nkt - 1 ||
         ((cls & 3) == TC_BOUNDARY && mask_mode != MASK_NONE);
}

// p = exp2(s') packed to bf16 as the PV operand; returns the lane's sum of
// the rounded p (bf16 pair dot products with ones, fp32 accumulation).
__device__ __forceinline__ float exp_pack(const f32x16 (&s)[2], b8v (&pb)[4]) {
#pragma unroll
  for (int bk = 0; bk < 2; ++bk)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      pb[2 * bk + (r >> 3)][r & 7] = (__bf16)__builtin_amdgcn_exp2f(s[bk][r]);
  const b2v one = {(__bf16)1.f, (__bf16)1.f};
  float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[ks], pb[ks], 0, 1), one, ps0,
                                          false);
    ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[ks], pb[ks], 2, 3), one, ps1,
                                          false);
    ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[ks], pb[ks], 4, 5), one, ps0,
                                          false);
    ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[ks], pb[ks], 6, 7), one, ps1,
                                          false);
  }
  return ps0 + ps1;
}

// Partner lane (l ^ 32) exchange as one VALU op: after the swap the two
// results hold this lane's and the partner's value, in lane-half order.
__device__ __forceinline__ float max_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ void reference_pv(const Tctx& c, const uint16_t* vs, f32x16 (&s)[2],
                                             b8v (&pb)[4], float psum, RowState& st);

__device__ __forceinline__ void softmax_pv_any(const Tctx& c, int j, int mask_mode,
                                               const uint16_t* vs, f32x16 (&s)[2],
                                               RowState& st) {
  const int cls = tile_cls_of(c, j);
  if (tile_needs_mask(c, j, cls, mask_mode)) mask_scores(c, j, cls, mask_mode, s);
  b8v pb[4];
  const float psum = exp_pack(s, pb);
  reference_pv(c, vs, s, pb, psum, st);
}

// After the exp: move the reference where a row needs it (rare), then the
// row sum and O^T += V^T P^T.
__device__ __forceinline__ void reference_pv(const Tctx& c, const uint16_t* vs, f32x16 (&s)[2],
                                             b8v (&pb)[4], float psum, RowState& st) {
  const bool need = !(psum <= kSumMax) || st.m == -INFINITY;
  if (__any(need)) {
    // Rare: move the reference of the rows that need it to their tile max.
    // Both lanes of a row take the same decision from exchanged values.
    float mt = -INFINITY;
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[bk][r]);
    mt = max_with_partner(mt);
    const bool grow = max_with_partner(need ? 1.f : 0.f) > 0.f && mt > -INFINITY;
    const float delta = grow ? mt : 0.f;
    const float alpha = grow ? (st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(-mt)) : 1.f;
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc[i][r] *= alpha;
    if (grow) st.m = (st.m == -INFINITY ? 0.f : st.m) + mt;
    const float nm = st.m == -INFINITY ? 0.f : -st.m;
#pragma unroll
    for (int r = 0; r < 16; ++r) st.negm[r] = nm;
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[bk][r] -= delta;
    psum = exp_pack(s, pb);
  }
  st.l += psum;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const uint16_t* vrow = vs + (32 * db + c.l32) * PF_BN;
    const int y = vswz(c.l32);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *(const b8v*)(vrow + 8 * ((2 * ks + c.hh) ^ y)), pb[ks], st.acc[db], 0, 0, 0);
  }
}

// A tile no mask can touch (all-remote, or wholly below the causal diagonal
// in a local or plain walk), scheduled by hand: the key operands of the first
// 32-key block are read together and block 1's are read while block 0's
// MFMAs run; block 1's MFMAs run under block 0's exponentials and the first
// value operands are read then; the PV product reads the operands of its
// next k-step while the current one runs. So no MFMA waits for a read issued
// just before it. The wave raises its issue priority over its MFMA phases and
// drops it for the second block's exponentials, so the other wave on the
// SIMD gets the issue slots while this one has only vector work. Same
// operations, in the same order per value, as qk_lds followed by
// softmax_pv_any.
__device__ __forceinline__ void tile_nomask(const Tctx& c, const uint16_t* ks, const uint16_t* vs,
                                            const h8v (&q)[8], RowState& st) {
  const int x = kswz(c.l32), y = vswz(c.l32);
  const uint16_t* kr0 = ks + c.l32 * PF_D;
  const uint16_t* kr1 = ks + (32 + c.l32) * PF_D;
  auto vop = [&](int db, int kk) __attribute__((always_inline)) -> b8v {
    return *(const b8v*)(vs + (32 * db + c.l32) * PF_BN + 8 * ((2 * kk + c.hh) ^ y));
  };
  h8v ka[8], kb[8];
  f32x16 s[2];
  __builtin_amdgcn_s_setprio(1);
  // ---- block 0
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) ka[cc] = *(const h8v*)(kr0 + 8 * ((2 * cc + c.hh) ^ x));
  s[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[0], q[0], st.negm, 0, 0, 0);
#pragma unroll
  for (int cc = 1; cc < 8; ++cc)
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[cc], q[cc], s[0], 0, 0, 0);
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) kb[cc] = *(const h8v*)(kr1 + 8 * ((2 * cc + c.hh) ^ x));
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // block 0's reads
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // an MFMA of block 0
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // a read for block 1
  }
  __builtin_amdgcn_sched_barrier(0);
  // ---- block 1, block 0's exponentials, the first value operands
  const b2v one = {(__bf16)1.f, (__bf16)1.f};
  b8v pb[4];
  float ps0 = 0.f, ps1 = 0.f;
  auto expb = [&](int bk) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      pb[2 * bk + (r >> 3)][r & 7] = (__bf16)__builtin_amdgcn_exp2f(s[bk][r]);
#pragma unroll
    for (int ks2 = 2 * bk; ks2 < 2 * bk + 2; ++ks2) {
      ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[ks2], pb[ks2], 0, 1), one,
                                            ps0, false);
      ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[ks2], pb[ks2], 2, 3), one,
                                            ps1, false);
      ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[ks2], pb[ks2], 4, 5), one,
                                            ps0, false);
      ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[ks2], pb[ks2], 6, 7), one,
                                            ps1, false);
    }
  };
  b8v vc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) vc[db] = vop(db, 0);
  s[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kb[0], q[0], st.negm, 0, 0, 0);
#pragma unroll
  for (int cc = 1; cc < 8; ++cc)
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kb[cc], q[cc], s[1], 0, 0, 0);
  expb(0);
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // value operands of k-step 0
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  expb(1);
  float psum = ps0 + ps1;
  // ---- reference (rare), row sum, O^T += V^T P^T
  const bool need = !(psum <= kSumMax) || st.m == -INFINITY;
  if (__any(need)) {
    float mt = -INFINITY;
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[bk][r]);
    mt = max_with_partner(mt);
    const bool grow = max_with_partner(need ? 1.f : 0.f) > 0.f && mt > -INFINITY;
    const float delta = grow ? mt : 0.f;
    const float alpha = grow ? (st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(-mt)) : 1.f;
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc[i][r] *= alpha;
    if (grow) st.m = (st.m == -INFINITY ? 0.f : st.m) + mt;
    const float nm = st.m == -INFINITY ? 0.f : -st.m;
#pragma unroll
    for (int r = 0; r < 16; ++r) st.negm[r] = nm;
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[bk][r] -= delta;
    psum = exp_pack(s, pb);
  }
  st.l += psum;
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    b8v vn[4];
    if (kk < 3) {
#pragma unroll
      for (int db = 0; db < 4; ++db) vn[db] = vop(db, kk + 1);
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
      st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vc[db], pb[kk], st.acc[db], 0, 0, 0);
    if (kk < 3) {
#pragma unroll
      for (int db = 0; db < 4; ++db) vc[db] = vn[db];
    }
  }
  __builtin_amdgcn_s_setprio(0);
}

// The same mask-free tile with one reference check per 32-key block: block
// 0's half of the PV product is issued right after its check, under block
// 1's exponentials. Equal to tile_nomask whenever the reference does not
// move in the tile; when it moves at block 1, block 0's products already in
// the accumulator are rescaled with it (the online-softmax update), equal up
// to rounding. The plain pass takes this step: compiled into that kernel it
// ran faster than tile_nomask (121.5 -> 119.3 ms at 128K, A/B), compiled into
// the fused kernel slower (120.3 -> 121.2 ms), with the same instructions per
// tile in both kernels.
__device__ __forceinline__ void tile_nomask_split(const Tctx& c, const uint16_t* ks,
                                                  const uint16_t* vs, const h8v (&q)[8],
                                                  RowState& st) {
  const int x = kswz(c.l32), y = vswz(c.l32);
  const uint16_t* kr0 = ks + c.l32 * PF_D;
  const uint16_t* kr1 = ks + (32 + c.l32) * PF_D;
  auto vop = [&](int db, int kk) __attribute__((always_inline)) -> b8v {
    return *(const b8v*)(vs + (32 * db + c.l32) * PF_BN + 8 * ((2 * kk + c.hh) ^ y));
  };
  h8v ka[8], kb[8];
  f32x16 s[2];
  __builtin_amdgcn_s_setprio(1);
  // ---- block 0
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) ka[cc] = *(const h8v*)(kr0 + 8 * ((2 * cc + c.hh) ^ x));
  s[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[0], q[0], st.negm, 0, 0, 0);
#pragma unroll
  for (int cc = 1; cc < 8; ++cc)
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[cc], q[cc], s[0], 0, 0, 0);
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) kb[cc] = *(const h8v*)(kr1 + 8 * ((2 * cc + c.hh) ^ x));
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // block 0's reads
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // an MFMA of block 0
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // a read for block 1
  }
  __builtin_amdgcn_sched_barrier(0);
  // ---- block 1's scores under block 0's exponentials; first value operands
  const b2v one = {(__bf16)1.f, (__bf16)1.f};
  b8v pb[4];
  // p = exp2(s') of block bk into pb[2 bk], pb[2 bk + 1]; returns its sum
  auto expb = [&](int bk) __attribute__((always_inline)) -> float {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      pb[2 * bk + (r >> 3)][r & 7] = (__bf16)__builtin_amdgcn_exp2f(s[bk][r]);
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int ks2 = 2 * bk; ks2 < 2 * bk + 2; ++ks2) {
      ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[ks2], pb[ks2], 0, 1), one,
                                            ps0, false);
      ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[ks2], pb[ks2], 2, 3), one,
                                            ps1, false);
      ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[ks2], pb[ks2], 4, 5), one,
                                            ps0, false);
      ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[ks2], pb[ks2], 6, 7), one,
                                            ps1, false);
    }
    return ps0 + ps1;
  };
  // rare: move the reference of the rows that need it to the maximum of
  // block bk's shifted scores, rescale acc and l (O^T so far, this tile's
  // block 0 included when bk = 1), shift the scores not yet exponentiated
  // and redo block bk's exponentials
  auto reference = [&](int bk, bool need, float psum) __attribute__((always_inline)) -> float {
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[bk][r]);
    mt = max_with_partner(mt);
    const bool grow = max_with_partner(need ? 1.f : 0.f) > 0.f && mt > -INFINITY;
    const float delta = grow ? mt : 0.f;
    const float alpha = grow ? (st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(-mt)) : 1.f;
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc[i][r] *= alpha;
    if (grow) st.m = (st.m == -INFINITY ? 0.f : st.m) + mt;
    const float nm = st.m == -INFINITY ? 0.f : -st.m;
#pragma unroll
    for (int r = 0; r < 16; ++r) st.negm[r] = nm;
#pragma unroll
    for (int b = bk; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[b][r] -= delta;
    return grow ? expb(bk) : psum;
  };
  b8v vc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) vc[db] = vop(db, 0);
  s[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kb[0], q[0], st.negm, 0, 0, 0);
#pragma unroll
  for (int cc = 1; cc < 8; ++cc)
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kb[cc], q[cc], s[1], 0, 0, 0);
  float ps_a = expb(0);
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // value operands of k-step 0
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  {
    const bool need = !(ps_a <= kSumMax) || st.m == -INFINITY;
    if (__any(need)) ps_a = reference(0, need, ps_a);
  }
  st.l += ps_a;
  // ---- block 0's half of O^T += V^T P^T under block 1's exponentials
  b8v vn[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) vn[db] = vop(db, 1);
#pragma unroll
  for (int db = 0; db < 4; ++db)
    st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vc[db], pb[0], st.acc[db], 0, 0, 0);
#pragma unroll
  for (int db = 0; db < 4; ++db) vc[db] = vop(db, 2);
#pragma unroll
  for (int db = 0; db < 4; ++db)
    st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vn[db], pb[1], st.acc[db], 0, 0, 0);
  float ps_b = expb(1);
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // value operands of k-step 1
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // value operands of k-step 2
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  {
    const bool need = !(ps_b <= kSumMax) || st.m == -INFINITY;
    if (__any(need)) ps_b = reference(1, need, ps_b);
  }
  st.l += ps_b;
  // ---- block 1's half
#pragma unroll
  for (int db = 0; db < 4; ++db) vn[db] = vop(db, 3);
#pragma unroll
  for (int db = 0; db < 4; ++db)
    st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vc[db], pb[2], st.acc[db], 0, 0, 0);
#pragma unroll
  for (int db = 0; db < 4; ++db)
    st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vn[db], pb[3], st.acc[db], 0, 0, 0);
  __builtin_amdgcn_s_setprio(0);
}

// One key tile from stage (kc, vc) while the next one (if any) streams into
// (kn, vn). NOMASK: a tile no mask can touch, on the hand-scheduled step
// (the same operations per value as the generic one).
template <bool NOMASK>
__device__ __forceinline__ void tile_step(const Tctx& c, int j, int nxt, bool nrem, int mask_mode,
                                          const h8v (&q)[8], const uint16_t* kc,
                                          const uint16_t* vc, uint16_t* kn, uint16_t* vn,
                                          RowState& st) {
  if (nxt >= 0) tile_dma(c, nxt, nrem, kn, vn);
  if constexpr (NOMASK) {
    tile_nomask(c, kc, vc, q, st);
  } else {
    f32x16 s[2];
    qk_lds(c, kc, q, st.negm, s);
    softmax_pv_any(c, j, mask_mode, vc, s, st);
  }
  tile_sync();
}
// Double-buffered walk over key tiles [j0, j1) whose LDS key tiles hold the
// rotation `rem_src` (remote tiles: remapped keys). `next_after` is the tile
// to prefetch after the last one (-1: none) and `next_rem` its rotation, so
// segments chain in any order. `stg` is the LDS stage holding tile j0.
// NOMASK: every tile of the segment is mask-free (see tile_step).
template <bool NOMASK = false>
__device__ __forceinline__ void walk(const Tctx& c, int j0, int j1, bool rem_src, int next_after,
                                     bool next_rem, int mask_mode, const h8v (&q)[8],
                                     const Stages& S, int& stg, RowState& st) {
  for (int j = j0; j < j1; ++j) {
    const int nxt = j + 1 < j1 ? j + 1 : next_after;
    const bool nrem = j + 1 < j1 ? rem_src : next_rem;
    tile_step<NOMASK>(c, j, nxt, nrem, mask_mode, q, stg ? S.k1 : S.k0, stg ? S.v1 : S.v0,
                      stg ? S.k0 : S.k1, stg ? S.v0 : S.v1, st);
    stg ^= 1;
  }
}
// Boundary tiles of the fused pass: the LDS key tile holds the absolute
// keys; the remapped scores come from the global key tile.
__device__ __forceinline__ void boundary_step(const Tctx& c, int j, int nxt, const h8v (&qa)[8],
                                              const h8v (&qr)[8], const uint16_t* kc,
                                              const uint16_t* vc, uint16_t* kn, uint16_t* vn,
                                              RowState& st) {
  if (nxt >= 0) tile_dma(c, nxt, false, kn, vn);
  f32x16 s[2];
  qk_lds(c, kc, qa, st.negm, s);
  boundary_select(c, j, qr, st.negm, s);
  softmax_pv_any(c, j, MASK_NONE, vc, s, st);
  tile_sync();
}
__device__ __forceinline__ void walk_boundary(const Tctx& c, int j0, int j1, int next_after,
                                              const h8v (&qa)[8], const h8v (&qr)[8],
                                              const Stages& S, int& stg, RowState& st) {
  for (int j = j0; j < j1; ++j) {
    const int nxt = j + 1 < j1 ? j + 1 : next_after;
    boundary_step(c, j, nxt, qa, qr, stg ? S.k1 : S.k0, stg ? S.v1 : S.v0, stg ? S.k0 : S.k1,
                  stg ? S.v0 : S.v1, st);
    stg ^= 1;
  }
}
// RoPE(x_q, p) of the lane's raw query row as the fp16 QK^T operand. The lane
// holds d = 16c + 8hh + j (c = 0..7, j = 0..7); the rotation pairs (d, d+64)
// are chunks (c, c+4) of the same lane. w2pi: omega_i / (2 pi) in LDS.
// Sets JL_FLAG_Q_RANGE in *flags when an operand is not a finite fp16 value.
__device__ __forceinline__ void rotate_query(const u32x4 (&raw)[8], double p, int hh,
                                             const double* w2pi, h8v (&out)[8], int* flags) {
  uint32_t nonfinite = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x0 = bf16_lane(raw[c], j), x1 = bf16_lane(raw[c + 4], j);
      float cs, sn;
      rope_cs_turns(p, w2pi[16 * c + 8 * hh + j], cs, sn);
      const _Float16 y0 = (_Float16)(x0 * cs - x1 * sn), y1 = (_Float16)(x0 * sn + x1 * cs);
      out[c][j] = y0;
      out[c + 4][j] = y1;
      // (bit casts of scalars: a bit cast of a vector element expression
      // reads element 0 whatever the index)
      nonfinite |= f16_nonfinite(__builtin_bit_cast(uint16_t, y0)) |
                   f16_nonfinite(__builtin_bit_cast(uint16_t, y1));
    }
  }
  if (nonfinite) atomicOr(flags, JL_FLAG_Q_RANGE);
}

template <int PASS>
__global__ void __launch_bounds__(256, 2) prefill_bf16_kernel(PfArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks0[PF_BN * PF_D];
  __shared__ __attribute__((aligned(16))) uint16_t Ks1[PF_BN * PF_D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs0[PF_D * PF_BN];
  __shared__ __attribute__((aligned(16))) uint16_t Vs1[PF_D * PF_BN];
  __shared__ double w2pi_s[PF_D / 2];  // omega_i / (2 pi)

  const int Hq = a.Hq, Hkv = a.Hkv;
  // ---- work item: (schedule slot, query head); XCD-aware head grouping
  int slot, head;
  {
    const int w = blockIdx.x;
    if ((Hq & 7) == 0) {
      const int hpx = Hq >> 3, k = w >> 3;
      slot = k / hpx;
      head = (w & 7) * hpx + k % hpx;
    } else {
      slot = w / Hq;
      head = w % Hq;
    }
  }
  const int* __restrict__ hdr = a.hdr;
  if (slot >= hdr[0]) return;
  if (threadIdx.x < PF_D / 2) w2pi_s[threadIdx.x] = a.fr.w(threadIdx.x) * kInvTwoPi;
  const int* __restrict__ tbase = a.tbase;
  int t;
  {
    int lo = 0, hi = hdr[1] - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (tbase[mid] <= slot) hi = mid; else lo = mid + 1;
    }
    t = lo;
  }
  const SeqInfo sq = a.seqs[a.order[slot - tbase[t]]];
  const int g = head / (Hq / Hkv);
  const int R = a.R;

  Tctx c;
  c.tid = threadIdx.x;
  c.hh = (c.tid & 63) >> 5;
  c.l32 = c.tid & 31;
  c.q0 = a.qoff + t * PF_BM;
  c.q1 = min(c.q0 + PF_BM, sq.len) - 1;
  c.len = sq.len;
  c.myq = c.q0 + (c.tid >> 6) * 32 + c.l32;
  c.nkt = c.q1 / PF_BN + 1;
  c.w0 = a.w0;
  c.R = R;
  c.kabs = a.kabs + ((int64_t)g * R + sq.pad_off) * PF_D;
  c.krem = a.krem + ((int64_t)g * R + sq.pad_off) * PF_D;
  c.vt = a.vt + (int64_t)g * PF_D * R + sq.pad_off;
  tile_dma_lanes<4>(c);
  const bool qvalid = c.myq < sq.len;

  // raw query row slice of this lane (zeros past the sequence end); re-read
  // before each rotation rather than kept live across the key loops
  const uint16_t* qp =
      a.xq + ((int64_t)(sq.start + (qvalid ? c.myq - a.qoff : 0)) * Hq + head) * PF_D + 8 * c.hh;
  auto rotq = [&](double p, h8v (&out)[8]) __attribute__((always_inline)) {
    u32x4 raw[8];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      raw[cc] = qvalid ? *(const u32x4*)(qp + 16 * cc) : u32x4{0, 0, 0, 0};
    rotate_query(raw, p, c.hh, w2pi_s, out, a.flags);
  };

  // first tile that is not all-remote, first tile that is all-local
  const int j_nr = c.q0 > c.w0 ? (c.q0 - c.w0) / PF_BN : 0;
  const int j_loc = c.q1 > c.w0 ? min(c.nkt, (c.q1 - c.w0 + PF_BN - 1) / PF_BN) : 0;
  constexpr bool kWin = PASS == PASS_IE_A || PASS == PASS_IE_B;  // B runs as C + remote keys
  const int jstart = kWin ? j_nr : 0;

  RowState st;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[i][r] = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) st.negm[r] = 0.f;
  st.m = -INFINITY;
  st.l = 0.f;
  int stg = 0;
  const Stages S{Ks0, Vs0, Ks1, Vs1};
  {
    // the first key tile: remapped keys for the remote phase of the fused
    // pass and for passes B/C, absolute otherwise
    const bool rem0 = (PASS == PASS_FUSED && jstart < j_nr) || PASS == PASS_IE_B;
    tile_dma(c, jstart, rem0, Ks0, Vs0);
  }
  tile_sync();  // also publishes w2pi_s

  if (PASS == PASS_FUSED) {
    const int jl0 = max(j_nr, j_loc);
    {
      h8v qr[8];
      rotq(remap_pos(c.myq, sq.G, a.cont), qr);
      // remote phase: remapped query against remapped key tiles (no mask
      // can apply: every key is more than w0 below every row)
      walk<true>(c, 0, j_nr, true, j_nr < c.nkt ? j_nr : -1, false, MASK_NONE, qr, S, stg, st);
      if (j_nr < j_loc) {  // boundary phase: both routes, element-wise select
        h8v qa[8];
        rotq(c.myq, qa);
        walk_boundary(c, j_nr, j_loc, jl0 < c.nkt ? jl0 : -1, qa, qr, S, stg, st);
      }
    }
    h8v qa[8];
    rotq(c.myq, qa);
    // local phase: absolute query against absolute key tiles; the tiles
    // wholly below the causal diagonal (every key <= q0 <= every row, inside
    // the sequence) need no mask
    const int jf = max(jl0, min(c.nkt, (c.q0 + 1) / PF_BN));
    walk<true>(c, jl0, jf, false, jf < c.nkt ? jf : -1, false, MASK_NONE, qa, S, stg, st);
    walk(c, jf, c.nkt, false, -1, false, MASK_NONE, qa, S, stg, st);
  } else if (PASS == PASS_PLAIN) {
    h8v qa[8];
    rotq(c.myq, qa);
    const int jf = min(c.nkt, (c.q0 + 1) / PF_BN);
    walk<true>(c, 0, jf, false, jf < c.nkt ? jf : -1, false, MASK_NONE, qa, S, stg, st);
    walk(c, jf, c.nkt, false, -1, false, MASK_NONE, qa, S, stg, st);
  } else if (PASS == PASS_IE_A) {
    h8v qa[8];
    rotq(c.myq, qa);
    walk(c, j_nr, c.nkt, false, -1, false, MASK_WINDOW, qa, S, stg, st);
  } else {
    // Passes C and B of Eq. 7 run this same code: the window keys first, in
    // the same order and with the same masks, so pass C's softmax state is a
    // bitwise prefix of pass B's; pass B (ie_remote = 1) then adds the remote
    // keys of the boundary tiles and the all-remote tiles. The shared window
    // part then cancels in W_B O_B - W_C O_C up to fp32 rounding.
    h8v qr[8];
    rotq(remap_pos(c.myq, sq.G, a.cont), qr);
    const int seg2 = j_nr < j_loc ? j_nr : (j_nr > 0 ? 0 : -1);
    walk(c, j_nr, c.nkt, true, a.ie_remote ? seg2 : -1, true, MASK_WINDOW, qr, S, stg, st);
    if (a.ie_remote) {
      walk(c, j_nr, j_loc, true, j_nr > 0 ? 0 : -1, true, MASK_REMOTE, qr, S, stg, st);
      walk<true>(c, 0, j_nr, true, -1, true, MASK_NONE, qr, S, stg, st);
    }
  }

  // ---- epilogue
  const float l_tot = st.l + xor32(st.l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (!qvalid) return;
  const int64_t row = (int64_t)(sq.start + c.myq - a.qoff);  // query row of the call
  if (PASS == PASS_IE_A || PASS == PASS_IE_B) {
    float* op = (float*)a.o + (row * Hq + head) * PF_D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *(float4*)(op + 32 * db + 8 * r4 + 4 * c.hh) =
            make_float4(st.acc[db][4 * r4] * inv, st.acc[db][4 * r4 + 1] * inv,
                        st.acc[db][4 * r4 + 2] * inv, st.acc[db][4 * r4 + 3] * inv);
  } else {
    uint16_t* op = (uint16_t*)a.o + (row * Hq + head) * PF_D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const uint32_t lo = (uint32_t)f32_to_bf16_bits(st.acc[db][4 * r4] * inv) |
                            ((uint32_t)f32_to_bf16_bits(st.acc[db][4 * r4 + 1] * inv) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_bits(st.acc[db][4 * r4 + 2] * inv) |
                            ((uint32_t)f32_to_bf16_bits(st.acc[db][4 * r4 + 3] * inv) << 16);
        *(uint2*)(op + 32 * db + 8 * r4 + 4 * c.hh) = make_uint2(lo, hi);
      }
  }
  if (a.lse && c.hh == 0) {
    const float lse = l_tot > 0.f ? (st.m + __log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
    a.lse[(int64_t)head * a.T + row] = lse;
  }
}

// ---------------------------------------------------------------------------
// Head-pair attention pass (fused and plain). Query heads 2p and 2p + 1 read
// the same KV head when Hq / Hkv is even, so one workgroup of 8 waves runs
// both on the same 128 query rows (waves 0-3: head 2p, waves 4-7: head
// 2p + 1) and every key / value tile staged in LDS feeds twice the MFMA work
// of the 4-wave pass. One workgroup per CU leaves LDS for three stages: the
// tile two ahead is in flight while a tile is computed. Both heads see the
// same tile classes (they depend on positions only), so all waves take the
// same path and the same barriers.
// ---------------------------------------------------------------------------
constexpr int PAIR_STAGES = 3;

// Tile j into a stage by 8 waves: transfer o = w + 8 i (i < 2) of each array.
// (kswz(r0 + 32 i) = kswz(r0), vswz(r0 + 64 i) = vswz(r0): a lane's swizzle
// is the same in both of its transfers of an array)
__device__ __forceinline__ void tile_dma8(const Tctx& c, int j, bool rem, uint16_t* ks,
                                          uint16_t* vs) {
  const int w = __builtin_amdgcn_readfirstlane(c.tid >> 6);
  const char* kg = (rem ? c.krem_l : c.kabs_l) + (int64_t)j * (PF_BN * PF_D * 2);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    __builtin_amdgcn_global_load_lds(
        (const void*)(kg + 32 * PF_D * 2 * i),
        (__attribute__((address_space(3))) void*)(ks + 512 * (w + 8 * i)), 16, 0, 0);
  const char* vg = c.vt_l + (int64_t)j * (PF_BN * 2);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    __builtin_amdgcn_global_load_lds(
        (const void*)(vg + c.vstep * i),
        (__attribute__((address_space(3))) void*)(vs + 512 * (w + 8 * i)), 16, 0, 0);
}

// End of a tile of the 3-stage walk: the tile after this one has landed
// (only the 4 transfers of the tile two ahead may still be in flight when
// `ahead`), this wave's LDS reads are done, then every wave is past this
// stage. No fence: it would also wait for the transfers two ahead.
__device__ __forceinline__ void pair_sync(bool ahead) {
  if (ahead) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int PASS>
__global__ void __launch_bounds__(512, 1) prefill_pair_kernel(PfArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks0[PF_BN * PF_D];
  __shared__ __attribute__((aligned(16))) uint16_t Ks1[PF_BN * PF_D];
  __shared__ __attribute__((aligned(16))) uint16_t Ks2[PF_BN * PF_D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs0[PF_D * PF_BN];
  __shared__ __attribute__((aligned(16))) uint16_t Vs1[PF_D * PF_BN];
  __shared__ __attribute__((aligned(16))) uint16_t Vs2[PF_D * PF_BN];
  __shared__ double w2pi_s[PF_D / 2];  // omega_i / (2 pi)

  const int Hq = a.Hq, Hkv = a.Hkv, npairs = Hq >> 1;
  // ---- work item: (schedule slot, head pair); XCD-aware pair grouping
  int slot, pair;
  {
    const int w = blockIdx.x;
    if ((npairs & 7) == 0) {
      const int hpx = npairs >> 3, k = w >> 3;
      slot = k / hpx;
      pair = (w & 7) * hpx + k % hpx;
    } else {
      slot = w / npairs;
      pair = w % npairs;
    }
  }
  const int* __restrict__ hdr = a.hdr;
  if (slot >= hdr[0]) return;
  if (threadIdx.x < PF_D / 2) w2pi_s[threadIdx.x] = a.fr.w(threadIdx.x) * kInvTwoPi;
  const int* __restrict__ tbase = a.tbase;
  int t;
  {
    int lo = 0, hi = hdr[1] - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (tbase[mid] <= slot) hi = mid; else lo = mid + 1;
    }
    t = lo;
  }
  const SeqInfo sq = a.seqs[a.order[slot - tbase[t]]];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int head = 2 * pair + (wave >> 2);
  const int g = (2 * pair) / (Hq / Hkv);
  const int R = a.R;

  Tctx c;
  c.tid = threadIdx.x;
  c.hh = (c.tid & 63) >> 5;
  c.l32 = c.tid & 31;
  c.q0 = a.qoff + t * PF_BM;
  c.q1 = min(c.q0 + PF_BM, sq.len) - 1;
  c.len = sq.len;
  c.myq = c.q0 + (wave & 3) * 32 + c.l32;
  c.nkt = c.q1 / PF_BN + 1;
  c.w0 = a.w0;
  c.R = R;
  c.kabs = a.kabs + ((int64_t)g * R + sq.pad_off) * PF_D;
  c.krem = a.krem + ((int64_t)g * R + sq.pad_off) * PF_D;
  c.vt = a.vt + (int64_t)g * PF_D * R + sq.pad_off;
  tile_dma_lanes<8>(c);
  const bool qvalid = c.myq < sq.len;

  const uint16_t* qp =
      a.xq + ((int64_t)(sq.start + (qvalid ? c.myq - a.qoff : 0)) * Hq + head) * PF_D + 8 * c.hh;
  auto rotq = [&](double p, h8v (&out)[8]) __attribute__((always_inline)) {
    u32x4 raw[8];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      raw[cc] = qvalid ? *(const u32x4*)(qp + 16 * cc) : u32x4{0, 0, 0, 0};
    rotate_query(raw, p, c.hh, w2pi_s, out, a.flags);
  };

  // first tile that is not all-remote, first tile that is all-local
  const int nkt = c.nkt;
  constexpr bool kIE = PASS == PASS_IE_A || PASS == PASS_IE_B;
  constexpr bool kRoute = PASS != PASS_PLAIN;
  const int j_nr = kRoute ? (c.q0 > c.w0 ? (c.q0 - c.w0) / PF_BN : 0) : 0;
  const int j_loc =
      kRoute ? (c.q1 > c.w0 ? min(nkt, (c.q1 - c.w0 + PF_BN - 1) / PF_BN) : 0) : 0;
  const int jl0 = max(j_nr, j_loc);
  // key tiles in walk order. Fused and plain: tile n at step n. Eq. 7 passes:
  // the window tiles j_nr .. nkt - 1 (window mask); pass B (ie_remote) then
  // the boundary tiles again (remote mask) and the all-remote tiles 0 ..
  // j_nr - 1, so pass C's softmax state is a bitwise prefix of pass B's.
  const bool ie_rem = PASS == PASS_IE_B && a.ie_remote;
  const int n1 = kIE ? nkt - j_nr : nkt;
  const int n2 = ie_rem ? max(j_loc - j_nr, 0) : 0;
  const int nwalk = n1 + n2 + (ie_rem ? j_nr : 0);
  auto tile_of = [&](int n) -> int {
    if (!kIE) return n;
    return n < n1 ? j_nr + n : n < n1 + n2 ? j_nr + (n - n1) : n - n1 - n2;
  };
  // remote tiles of the fused pass and every tile of passes B / C stage the
  // remapped keys
  auto rem_of = [&](int j) { return PASS == PASS_IE_B || (PASS == PASS_FUSED && j < j_nr); };
  auto kst = [&](int j) -> uint16_t* {  // stage of tile j: j mod 3
    const int s3 = j % PAIR_STAGES;
    return s3 == 0 ? Ks0 : s3 == 1 ? Ks1 : Ks2;
  };
  auto vst = [&](int j) -> uint16_t* {
    const int s3 = j % PAIR_STAGES;
    return s3 == 0 ? Vs0 : s3 == 1 ? Vs1 : Vs2;
  };

  RowState st;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[i][r] = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) st.negm[r] = 0.f;
  st.m = -INFINITY;
  st.l = 0.f;

  // the walk's first two tiles in flight; wait for them (and w2pi_s)
  tile_dma8(c, tile_of(0), rem_of(tile_of(0)), Ks0, Vs0);
  if (nwalk > 1) tile_dma8(c, tile_of(1), rem_of(tile_of(1)), Ks1, Vs1);
  __syncthreads();  // publishes w2pi_s (the fence also waits for both tiles)

  // one tile: prefetch j + 2 into the stage freed at the last barrier,
  // compute j, wait for j + 1. Boundary tiles get the remapped query through
  // qr_b; taking its address makes the compiler keep that array in private
  // memory (128 B per lane, written once per workgroup, re-read from cache
  // in the few boundary tiles), which leaves the registers to the main
  // loops. An LDS copy instead gave the same results and ran 1% slower.
  auto step = [&](int j, const h8v (&q)[8], const h8v* qr_b) __attribute__((always_inline)) {
    const bool ahead = j + 2 < nkt;
    if (ahead) tile_dma8(c, j + 2, rem_of(j + 2), kst(j + 2), vst(j + 2));
    f32x16 s[2];
    qk_lds(c, kst(j), q, st.negm, s);
    if (qr_b) boundary_select(c, j, *(const h8v(*)[8])qr_b, st.negm, s);
    softmax_pv_any(c, j, MASK_NONE, vst(j), s, st);
    pair_sync(ahead);
  };
  auto step_nomask = [&](int j, const h8v (&q)[8]) __attribute__((always_inline)) {
    const bool ahead = j + 2 < nkt;
    if (ahead) tile_dma8(c, j + 2, rem_of(j + 2), kst(j + 2), vst(j + 2));
    tile_nomask(c, kst(j), vst(j), q, st);
    pair_sync(ahead);
  };
  // tiles wholly below the causal diagonal: every key <= q0 <= every row of
  // the tile (and inside the sequence), so no mask can apply
  const int j_free = min(nkt, (c.q0 + 1) / PF_BN);
  if (PASS == PASS_FUSED) {
    {
      h8v qr[8];
      rotq(remap_pos(c.myq, sq.G, a.cont), qr);
      for (int j = 0; j < j_nr; ++j) step_nomask(j, qr);  // remote phase
      if (j_nr < j_loc) {                                    // boundary phase
        h8v qa[8];
        rotq(c.myq, qa);
        for (int j = j_nr; j < j_loc; ++j) step(j, qa, &qr[0]);
      }
    }
    h8v qa[8];
    rotq(c.myq, qa);
    // local phase: mask-free tiles, then the diagonal ones
    for (int j = jl0; j < j_free; ++j) step_nomask(j, qa);
    for (int j = max(jl0, j_free); j < nkt; ++j) step(j, qa, nullptr);
  } else if (kIE) {
    h8v q[8];
    rotq(PASS == PASS_IE_B ? remap_pos(c.myq, sq.G, a.cont) : (double)c.myq, q);
    // one loop per segment, so each has its mask mode at compile time
    auto step_ie = [&](int n, int j, auto mm) __attribute__((always_inline)) {
      const bool ahead = n + 2 < nwalk;
      if (ahead) {
        const int tn = tile_of(n + 2);
        tile_dma8(c, tn, rem_of(tn), kst(n + 2), vst(n + 2));
      }
      f32x16 s[2];
      qk_lds(c, kst(n), q, st.negm, s);
      softmax_pv_any(c, j, decltype(mm)::value, vst(n), s, st);
      pair_sync(ahead);
    };
    for (int n = 0; n < n1; ++n)
      step_ie(n, j_nr + n, std::integral_constant<int, MASK_WINDOW>{});
    for (int n = n1; n < n1 + n2; ++n)
      step_ie(n, j_nr + (n - n1), std::integral_constant<int, MASK_REMOTE>{});
    // the all-remote tiles (no mask can apply: see the fused pass) take the
    // hand-scheduled step, which performs the same operations per value
    for (int n = n1 + n2; n < nwalk; ++n) {
      const bool ahead = n + 2 < nwalk;
      if (ahead) {
        const int tn = tile_of(n + 2);
        tile_dma8(c, tn, rem_of(tn), kst(n + 2), vst(n + 2));
      }
      tile_nomask(c, kst(n), vst(n), q, st);
      pair_sync(ahead);
    }
  } else {
    // plain causal RoPE attention (the baseline): a mask-free step on every
    // tile below the diagonal (the per-block-check one, the faster of the
    // two in this kernel)
    h8v qa[8];
    rotq(c.myq, qa);
    for (int j = 0; j < j_free; ++j) {
      const bool ahead = j + 2 < nkt;
      if (ahead) tile_dma8(c, j + 2, false, kst(j + 2), vst(j + 2));
      tile_nomask_split(c, kst(j), vst(j), qa, st);
      pair_sync(ahead);
    }
    for (int j = j_free; j < nkt; ++j) step(j, qa, nullptr);
  }

  // ---- epilogue
  const float l_tot = st.l + xor32(st.l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (!qvalid) return;
  const int64_t row = (int64_t)(sq.start + c.myq - a.qoff);
  if constexpr (kIE) {  // Eq. 7 passes keep float32 partial outputs
    float* op = (float*)a.o + (row * Hq + head) * PF_D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *(float4*)(op + 32 * db + 8 * r4 + 4 * c.hh) =
            make_float4(st.acc[db][4 * r4] * inv, st.acc[db][4 * r4 + 1] * inv,
                        st.acc[db][4 * r4 + 2] * inv, st.acc[db][4 * r4 + 3] * inv);
  } else {
    uint16_t* op = (uint16_t*)a.o + (row * Hq + head) * PF_D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const uint32_t lo = (uint32_t)f32_to_bf16_bits(st.acc[db][4 * r4] * inv) |
                            ((uint32_t)f32_to_bf16_bits(st.acc[db][4 * r4 + 1] * inv) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_bits(st.acc[db][4 * r4 + 2] * inv) |
                            ((uint32_t)f32_to_bf16_bits(st.acc[db][4 * r4 + 3] * inv) << 16);
        *(uint2*)(op + 32 * db + 8 * r4 + 4 * c.hh) = make_uint2(lo, hi);
      }
  }
  if (a.lse && c.hh == 0) {
    const float lse = l_tot > 0.f ? (st.m + __log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
    a.lse[(int64_t)head * a.T + row] = lse;
  }
}

hipError_t launch_prefill_bf16(int pass, const void* xq, void* o, float* lse, int64_t T, int B,
                               int Hq, int Hkv, int64_t w0, int64_t qoff, float scale, int cont,
                               const RopeFreqs& fr, void* ws, const PrefillLayout& lay,
                               hipStream_t st) {
  char* w = (char*)ws;
  PfArgs a;
  a.xq = (const uint16_t*)xq;
  a.kabs = (const uint16_t*)(w + lay.kabs);
  a.krem = (const uint16_t*)(w + lay.krem);
  a.vt = (const uint16_t*)(w + lay.vt);
  a.o = o;
  a.lse = lse;
  a.seqs = (const SeqInfo*)(w + lay.seqs);
  a.hdr = (const int*)(w + lay.hdr);
  a.order = (const int*)(w + lay.tiles);
  a.tact = a.order + B;
  a.tbase = a.tact + (lay.max_tiles + 1);
  a.T = (int)T;
  a.R = (int)lay.R;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.w0 = (int)w0;
  a.qoff = (int)qoff;
  a.ie_remote = pass == PASS_IE_B;
  a.cont = cont;
  (void)scale;  // the score scale is carried by the key operands (pre-pass)
  a.fr = fr;
  a.flags = (int*)(w + lay.hdr) + kHdrFlags;
  const int64_t blocks = lay.max_tiles * Hq;
  if ((Hq / Hkv) % 2 == 0) {
    const dim3 grid((unsigned)(lay.max_tiles * (Hq / 2)));
    switch (pass) {
      case PASS_FUSED:
        hipLaunchKernelGGL(prefill_pair_kernel<PASS_FUSED>, grid, dim3(512), 0, st, a);
        break;
      case PASS_PLAIN:
        hipLaunchKernelGGL(prefill_pair_kernel<PASS_PLAIN>, grid, dim3(512), 0, st, a);
        break;
      case PASS_IE_A:
        hipLaunchKernelGGL(prefill_pair_kernel<PASS_IE_A>, grid, dim3(512), 0, st, a);
        break;
      default:  // passes B and C share one instantiation
        hipLaunchKernelGGL(prefill_pair_kernel<PASS_IE_B>, grid, dim3(512), 0, st, a);
        break;
    }
    return hipGetLastError();
  }
  switch (pass) {
    case PASS_FUSED:
      hipLaunchKernelGGL(prefill_bf16_kernel<PASS_FUSED>, dim3(blocks), dim3(256), 0, st, a);
      break;
    case PASS_PLAIN:
      hipLaunchKernelGGL(prefill_bf16_kernel<PASS_PLAIN>, dim3(blocks), dim3(256), 0, st, a);
      break;
    case PASS_IE_A:
      hipLaunchKernelGGL(prefill_bf16_kernel<PASS_IE_A>, dim3(blocks), dim3(256), 0, st, a);
      break;
    default:  // passes B and C share one instantiation (see the kernel)
      hipLaunchKernelGGL(prefill_bf16_kernel<PASS_IE_B>, dim3(blocks), dim3(256), 0, st, a);
      break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Device tile-class dump (same classifier and tile shape as the kernel).
// ---------------------------------------------------------------------------
__global__ void tile_dump_kernel(int L, int w0, int nq, int nk, int8_t* out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)nq * nk) return;
  const int i = (int)(idx / nk), j = (int)(idx % nk);
  const int q0 = i * PF_BM, q1 = min(q0 + PF_BM, L) - 1;
  const int k0 = j * PF_BN, k1 = min(k0 + PF_BN, L) - 1;
  out[idx] = (int8_t)tile_class(q0, q1, k0, k1, w0);
}

hipError_t launch_tile_dump(int64_t L, int64_t w0, int8_t* out, hipStream_t st) {
  const int nq = (int)((L + PF_BM - 1) / PF_BM), nk = (int)((L + PF_BN - 1) / PF_BN);
  const int64_t n = (int64_t)nq * nk;
  const int w0c = w0 > (int64_t)INT32_MAX ? INT32_MAX : (int)w0;
  hipLaunchKernelGGL(tile_dump_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     (int)L, w0c, nq, nk, out);
  return hipGetLastError();
}

}  // namespace jl
