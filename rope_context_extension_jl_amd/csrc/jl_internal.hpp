// Internal declarations shared by the libbifocal sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bifocal.h"

namespace jl {

// ---------------------------------------------------------------------------
// Tile classification from the routing condition of Eq. 1 (r9-hu digest,
// Method). Distance-only: the class never depends on G.
//   0 masked, 1 local, 2 remote, 3 boundary; +4 when the diagonal crosses.
// ---------------------------------------------------------------------------
enum TileClass : int { TC_MASKED = 0, TC_LOCAL = 1, TC_REMOTE = 2, TC_BOUNDARY = 3, TC_DIAG = 4 };

__host__ __device__ inline int tile_class(int64_t q0, int64_t q1, int64_t k0, int64_t k1,
                                          int64_t w0) {
  if (k0 > q1) return TC_MASKED;
  int c;
  if (q1 - k0 <= w0) c = TC_LOCAL;        // largest causal distance inside the window
  else if (q0 - k1 > w0) c = TC_REMOTE;   // smallest distance outside it
  else c = TC_BOUNDARY;
  if (k1 > q0) c += TC_DIAG;              // some pair has k > q
  return c;
}

// Eq. 2 in integer arithmetic: ceil(L / w_pre), at least 1, written so that
// no intermediate overflows for any L, w_pre >= 1.
__host__ __device__ inline int64_t group_size(int64_t L, int64_t w_pre) {
  const int64_t g = L / w_pre + (L % w_pre != 0);
  return g < 1 ? 1 : g;
}

// Rotary frequencies omega_i = theta^(-2i/d) = 2^(i * (-2 log2(theta) / d)),
// evaluated in float64 where they are used (one scalar travels in the kernel
// arguments instead of a table that lanes would index).
struct RopeFreqs {
  double nl2t;  // -2 * log2(theta) / d
  __host__ __device__ double w(int i) const { return exp2((double)i * nl2t); }
};
void make_freqs(RopeFreqs& f, int d, double theta);

// Word of the prefill workspace header (int32 index) that holds the range
// flags of the last call (JL_FLAG_* of bifocal.h); the plan kernel clears it.
constexpr int kHdrFlags = 3;

// Per-sequence record built on the device by the plan kernel.
struct SeqInfo {
  int start;    // first token (row of the packed [T, H, d] tensors)
  int len;      // tokens in the sequence
  int G;        // Eq. 2 group size from this sequence's length
  int pad_off;  // first row of this sequence in the 64-row padded workspace layout
};

// Prefill tile shapes of the bf16 MFMA kernel.
constexpr int PF_BM = 128;   // query rows per workgroup (4 waves x 32)
constexpr int PF_BN = 64;    // keys per tile
constexpr int PF_D = 128;    // head dim
// fp32 VALU kernel.
constexpr int PF32_BM = 64;
constexpr int PF32_BN = 32;

enum Pass : int { PASS_FUSED = 0, PASS_PLAIN = 1, PASS_IE_A = 2, PASS_IE_B = 3, PASS_IE_C = 4 };

// Workspace carving shared by the API and the kernels' launchers.
struct PrefillLayout {
  size_t hdr, seqs, tiles, kabs, krem, vt, ie_o, ie_lse, ie_ratio, total;
  int64_t R;          // padded rows per KV head
  int64_t max_tiles;  // upper bound on query tiles
};
PrefillLayout prefill_layout(int64_t T, int B, int Hq, int Hkv, int d, int dtype, int mode);

// ---------------------------------------------------------------------------
// Launchers (return hipError_t of the launch).
// ---------------------------------------------------------------------------
hipError_t launch_rope_apply(void* x, int64_t T, int H, int d, const int32_t* cu, int B,
                             int64_t pos_offset, const RopeFreqs& fr, int is_f32,
                             hipStream_t st);

// qoff: position of the first query row of a single sequence (0 = all rows
// are queries); the query tiles then cover rows qoff .. T-1.
hipError_t launch_prefill_plan(const int32_t* cu, int B, int64_t T, int64_t qoff, int64_t w_pre,
                               int bm, void* ws, const PrefillLayout& lay, hipStream_t st);

// from_abs: the keys are already rotated at their absolute positions.
// kscale multiplies the fp16 key operands (not the bf16 cache written).
// cont (here and below): remote positions are the real numbers x / G
// instead of floor(x / G) (the continuous-interpolation remote map).
hipError_t launch_prefill_prep_bf16(const void* xk, const void* v, void* kcache_out, int64_t T,
                                    int B, int Hkv, int need_rem, int from_abs, float kscale,
                                    int cont, const RopeFreqs& fr, void* ws,
                                    const PrefillLayout& lay, hipStream_t st);

hipError_t launch_prefill_bf16(int pass, const void* xq, void* o, float* lse, int64_t T, int B,
                               int Hq, int Hkv, int64_t w0, int64_t qoff, float scale, int cont,
                               const RopeFreqs& fr, void* ws, const PrefillLayout& lay,
                               hipStream_t st);

hipError_t launch_prefill_prep_f32(const void* xk, void* kcache_out, int64_t T, int B, int Hkv,
                                   int d, int need_rem, int cont, const RopeFreqs& fr, void* ws,
                                   const PrefillLayout& lay, hipStream_t st);

hipError_t launch_prefill_f32(int pass, const void* xq, const void* v, void* o, float* lse,
                              int64_t T, int B, int Hq, int Hkv, int d, int64_t w0, float scale,
                              int cont, const RopeFreqs& fr, void* ws, const PrefillLayout& lay,
                              hipStream_t st);

hipError_t launch_ie_merge(void* o, float* lse, int out_f32, int64_t T, int Hq, int d, void* ws,
                           const PrefillLayout& lay, hipStream_t st);

hipError_t launch_decode(const void* xq, const void* kc, const void* vc, void* o, float* lse,
                         int64_t pos, int Hq, int Hkv, int d, int64_t w0, int64_t G, float scale,
                         const RopeFreqs& fr, int plain, int cont, int is_f32, int kps,
                         void* ws, hipStream_t st);

// Batched decode: sequence b's query is row b of xq [B, Hq, d], its keys
// 0 .. positions[b] sit at cache rows starts[b] + k; `splits` splits of `kps`
// keys each cover max_keys keys (the partials, at ws, are
// [B, Hq, splits, d + 2]). bf16: base (int32 [B + 1], device) receives the
// work list and grid_wg workgroups walk it.
hipError_t launch_decode_batch(const void* xq, const void* kc, const void* vc, void* o, float* lse,
                               const int32_t* positions, const int32_t* starts, int B,
                               int64_t max_keys, int64_t cap_rows, int Hq, int Hkv, int d,
                               int64_t w0, int64_t w_pre, float scale, const RopeFreqs& fr,
                               int plain, int cont, int is_f32, int splits, int kps, void* ws,
                               int* base, int grid_wg, hipStream_t st);

hipError_t launch_tile_dump(int64_t L, int64_t w0, int8_t* out, hipStream_t st);

// variant 0: grid-stride 16-byte loads, 4 in flight per thread; 1: 32 KiB
// chunks per workgroup, 8 nontemporal loads in flight per thread; 2: 64 KiB
// chunks by direct global -> LDS transfers; 3: variant 1 without and 4:
// variant 2 with the nontemporal hint.
hipError_t launch_calib_read(const void* src, size_t bytes, uint32_t* sink, int blocks,
                             int variant, hipStream_t st);
hipError_t launch_calib_mfma(float* sink, int blocks, int iters, hipStream_t st);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
#ifdef __HIPCC__
constexpr double kTwoPi = 6.283185307179586476925286766559;
constexpr double kInvTwoPi = 0.15915494309189533576888376337251;

// cos/sin of p * w: the product and its reduction modulo 2*pi are done in
// float64 (|p*w| reaches ~1.3e5 rad at 128K positions, where a float32
// product alone would be off by ~1e-2 rad); sin/cos of the reduced angle in
// float32.
__device__ inline void rope_cs(double p, double w, float& c, float& s) {
  double a = p * w;
  double n = __builtin_rint(a * kInvTwoPi);
  double r = __builtin_fma(-n, kTwoPi, a);
  sincosf((float)r, &s, &c);
}

// Same rotation with the angle in turns: t = p * (w / 2pi) is formed and
// reduced to [-1/2, 1/2] in float64, then the hardware sine and cosine (which
// take turns) finish it in float32. For paths whose operands are rounded to
// 16-bit floats. w2pi = w / (2 pi).
__device__ inline void rope_cs_turns(double p, double w2pi, float& c, float& s) {
  const double t = p * w2pi;
  const float f = (float)(t - __builtin_rint(t));
  s = __builtin_amdgcn_sinf(f);
  c = __builtin_amdgcn_cosf(f);
}

// Remote position f(x) of Eq. 1: floor(x / G), the aliasing map, or with
// cont set the real number x / G (continuous frequency interpolation by the
// same factor: a rotation by (x / G) w is a rotation by x at frequency w / G).
__device__ inline double remap_pos(int x, int G, int cont) {
  return cont ? (double)x / (double)G : (double)(x / G);
}

__device__ inline float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// Element j (0..7) of eight bf16 values packed in a 16-byte vector, as float.
typedef uint32_t jl_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float bf16_lane(const jl_u32x4& v, int j) {
  const uint32_t w = v[j >> 1];
  return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
}

__device__ inline uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint16_t, h);
}
__device__ inline uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
// 1 when the fp16 bit pattern is an infinity or a NaN (all exponent bits set).
__device__ __forceinline__ uint32_t f16_nonfinite(uint16_t b) {
  return (b & 0x7c00u) == 0x7c00u ? 1u : 0u;
}
#endif

}  // namespace jl
