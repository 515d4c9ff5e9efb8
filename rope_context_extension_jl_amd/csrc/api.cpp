// C ABI of libbifocal: argument validation, workspace layout and dispatch.
// Every check runs on the host before any launch (see include/bifocal.h).
#include "../../include/bifocal.h"

#include <math.h>
#include <string.h>

#include <mutex>

#include "jl_internal.hpp"

namespace jl {

static thread_local int g_last_hip_error = 0;

static int hip_status(hipError_t e) {
  if (e == hipSuccess) return JL_OK;
  g_last_hip_error = (int)e;
  return JL_EHIP;
}

void make_freqs(RopeFreqs& f, int d, double theta) { f.nl2t = -2.0 * log2(theta) / (double)d; }

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

PrefillLayout prefill_layout(int64_t T, int B, int Hq, int Hkv, int d, int dtype, int mode) {
  PrefillLayout L{};
  const int bm = dtype == JL_BF16 ? PF_BM : PF32_BM;
  // Every sequence starts on a 64-row boundary of the padded key layout.
  L.R = ((T + 63) / 64) * 64 + 64 * (int64_t)B;
  L.max_tiles = (T + bm - 1) / bm + B;
  const size_t elem = dtype == JL_BF16 ? 2 : 4;
  size_t off = 0;
  L.hdr = off;   off += 256;
  L.seqs = off;  off += align256((size_t)B * sizeof(SeqInfo));
  // tile schedule: sorted sequence order [B], per-depth active counts and
  // bases [max_tiles + 1] each (see the plan kernel).
  L.tiles = off; off += align256(((size_t)B + 2 * ((size_t)L.max_tiles + 1)) * sizeof(int));
  L.kabs = off;  off += align256((size_t)Hkv * L.R * d * elem);
  if (mode == JL_MODE_PLAIN) {
    L.krem = L.kabs;
  } else {
    L.krem = off; off += align256((size_t)Hkv * L.R * d * elem);
  }
  if (dtype == JL_BF16) {
    L.vt = off; off += align256((size_t)Hkv * L.R * d * 2);
  } else {
    L.vt = L.kabs;
  }
  L.ie_o = L.ie_lse = L.ie_ratio = off;
  if (mode == JL_MODE_IE) {
    L.ie_o = off;     off += align256(3 * (size_t)T * Hq * d * 4);
    L.ie_lse = off;   off += align256(3 * (size_t)T * Hq * 4);
    L.ie_ratio = off; off += align256((size_t)T * Hq * 4);
  }
  L.total = off;
  return L;
}

}  // namespace jl

using namespace jl;

extern "C" {

int64_t jl_group_size(int64_t L, int64_t w_pre) {
  if (L < 1 || w_pre < 1) return JL_EINVAL;
  return jl::group_size(L, w_pre);
}

int jl_tile_class(int64_t q0, int64_t q1, int64_t k0, int64_t k1, int64_t w0) {
  if (q0 < 0 || k0 < 0 || q1 < q0 || k1 < k0 || w0 < 0) return JL_EINVAL;
  return jl::tile_class(q0, q1, k0, k1, w0);
}

int jl_prefill_tile_shape(jl_dtype dt, int d, int* bm, int* bn) {
  if (!bm || !bn) return JL_EINVAL;
  if (dt == JL_BF16 && d == PF_D) {
    *bm = PF_BM;
    *bn = PF_BN;
    return JL_OK;
  }
  if (dt == JL_FP32 && (d == 64 || d == 128)) {
    *bm = PF32_BM;
    *bn = PF32_BN;
    return JL_OK;
  }
  return JL_EUNSUPPORTED;
}

int jl_rope_apply(void* x, int64_t T, int H, int d, const int32_t* cu_seqlens, int B,
                  int64_t pos_offset, double theta, jl_dtype dt, void* stream) {
  if (T < 0 || H < 1 || d < 2 || d > 256 || (d & 1) || pos_offset < 0 || !(theta > 1.0))
    return JL_EINVAL;
  if (dt != JL_BF16 && dt != JL_FP32) return JL_EINVAL;
  if (d % 16) return JL_EUNSUPPORTED;
  if (cu_seqlens && B < 1) return JL_EINVAL;
  if (T == 0) return JL_OK;
  if (!x) return JL_EINVAL;
  if (T > (int64_t)INT32_MAX || (double)T * H * d > 9.0e15) return JL_EINVAL;
  RopeFreqs fr;
  make_freqs(fr, d, theta);
  return hip_status(launch_rope_apply(x, T, H, d, cu_seqlens, cu_seqlens ? B : 1, pos_offset, fr,
                                      dt == JL_FP32, (hipStream_t)stream));
}

// The remote-map flag rides in the mode argument; the rest is the mode proper.
static jl_mode strip_remap(jl_mode mode, int* cont) {
  const int m = (int)mode;
  if (cont) *cont = (m & JL_REMAP_CONTINUOUS) ? 1 : 0;
  return (jl_mode)(m & ~JL_REMAP_CONTINUOUS);
}

// Head counts and head dims any entry point or size query accepts. With
// T, capacity <= 2^31, heads <= 2^16 and d <= 256 every byte count below
// stays far inside size_t.
constexpr int kMaxHeads = 1 << 16;
static bool heads_ok(int Hq, int Hkv) {
  return Hkv >= 1 && Hq >= Hkv && Hq <= kMaxHeads && Hq % Hkv == 0;
}
static bool dim_ok(int d) { return d >= 2 && d <= 256 && d % 2 == 0; }

static bool prefill_shape_ok(int64_t T, int B, int Hq, int Hkv, int d, jl_dtype dt, jl_mode mode) {
  if (T < 0 || B < 1 || B > 4096 || !heads_ok(Hq, Hkv) || !dim_ok(d)) return false;
  if (T > (int64_t)INT32_MAX / 2) return false;
  if (dt != JL_BF16 && dt != JL_FP32) return false;
  if (mode != JL_MODE_FUSED && mode != JL_MODE_IE && mode != JL_MODE_PLAIN) return false;
  return true;
}

size_t jl_prefill_workspace_size(int64_t T, int B, int Hq, int Hkv, int d, jl_dtype dt,
                                 jl_mode mode) {
  mode = strip_remap(mode, nullptr);
  if (!prefill_shape_ok(T, B, Hq, Hkv, d, dt, mode)) return 0;
  return prefill_layout(T, B, Hq, Hkv, d, dt, mode).total;
}

size_t jl_prefill_ie_ratio_offset(int64_t T, int B, int Hq, int Hkv, int d, jl_dtype dt) {
  if (!prefill_shape_ok(T, B, Hq, Hkv, d, dt, JL_MODE_IE)) return 0;
  return prefill_layout(T, B, Hq, Hkv, d, dt, JL_MODE_IE).ie_ratio;
}

int jl_bifocal_prefill_timed(const void* xq, const void* xk, const void* v, void* o, float* lse,
                             void* kcache_out, const int32_t* cu_seqlens, int B, int64_t T,
                             int Hq, int Hkv, int d, int64_t w0, int64_t w_pre, double theta,
                             float scale, jl_dtype dt, jl_mode mode, void* workspace,
                             size_t ws_bytes, void* stream, void* ev_begin, void* ev_end) {
  int cont;
  mode = strip_remap(mode, &cont);
  if (!cu_seqlens && B != 1) return JL_EINVAL;
  if (!prefill_shape_ok(T, B, Hq, Hkv, d, dt, mode)) return JL_EINVAL;
  if (w0 < 0 || w_pre < 1 || !(theta > 1.0) || !(scale == scale)) return JL_EINVAL;
  if (w0 > (int64_t)INT32_MAX) w0 = INT32_MAX;  // every pair of a 32-bit sequence is local
  if (dt == JL_BF16 && d != PF_D) return JL_EUNSUPPORTED;
  if (dt == JL_FP32 && d != 64 && d != 128) return JL_EUNSUPPORTED;
  if (T == 0) return JL_OK;
  if (!xq || !xk || !v || !o) return JL_EINVAL;
  const PrefillLayout lay = prefill_layout(T, B, Hq, Hkv, d, dt, mode);
  if (!workspace || ws_bytes < lay.total) return JL_EWORKSPACE;
  if (((uintptr_t)workspace) & 255) return JL_EINVAL;
  const float sc = scale > 0.f ? scale : (float)(1.0 / sqrt((double)d));
  RopeFreqs fr;
  make_freqs(fr, d, theta);
  hipStream_t st = (hipStream_t)stream;
  const int bm = dt == JL_BF16 ? PF_BM : PF32_BM;
  hipError_t e = launch_prefill_plan(cu_seqlens, B, T, 0, w_pre, bm, workspace, lay, st);
  if (e != hipSuccess) return hip_status(e);
  const int need_rem = mode != JL_MODE_PLAIN;
  if (dt == JL_BF16) {
    e = launch_prefill_prep_bf16(xk, v, kcache_out, T, B, Hkv, need_rem, 0,
                                 sc * 1.4426950408889634f, cont, fr, workspace, lay, st);
    if (e != hipSuccess) return hip_status(e);
    if (ev_begin && (e = hipEventRecord((hipEvent_t)ev_begin, st)) != hipSuccess)
      return hip_status(e);
    if (mode == JL_MODE_IE) {
      float* base_o = (float*)((char*)workspace + lay.ie_o);
      float* base_l = (float*)((char*)workspace + lay.ie_lse);
      const size_t on = (size_t)T * Hq * d, ln = (size_t)T * Hq;
      const int passes[3] = {PASS_IE_A, PASS_IE_B, PASS_IE_C};
      for (int i = 0; i < 3; ++i) {
        e = launch_prefill_bf16(passes[i], xq, base_o + i * on, base_l + i * ln, T, B, Hq, Hkv,
                                w0, 0, sc, cont, fr, workspace, lay, st);
        if (e != hipSuccess) return hip_status(e);
      }
      e = launch_ie_merge(o, lse, 0, T, Hq, d, workspace, lay, st);
    } else {
      e = launch_prefill_bf16(mode == JL_MODE_PLAIN ? PASS_PLAIN : PASS_FUSED, xq, o, lse, T, B,
                              Hq, Hkv, w0, 0, sc, cont, fr, workspace, lay, st);
    }
  } else {
    e = launch_prefill_prep_f32(xk, kcache_out, T, B, Hkv, d, need_rem, cont, fr, workspace, lay,
                                st);
    if (e != hipSuccess) return hip_status(e);
    if (ev_begin && (e = hipEventRecord((hipEvent_t)ev_begin, st)) != hipSuccess)
      return hip_status(e);
    if (mode == JL_MODE_IE) {
      float* base_o = (float*)((char*)workspace + lay.ie_o);
      float* base_l = (float*)((char*)workspace + lay.ie_lse);
      const size_t on = (size_t)T * Hq * d, ln = (size_t)T * Hq;
      const int passes[3] = {PASS_IE_A, PASS_IE_B, PASS_IE_C};
      for (int i = 0; i < 3; ++i) {
        e = launch_prefill_f32(passes[i], xq, v, base_o + i * on, base_l + i * ln, T, B, Hq, Hkv,
                               d, w0, sc, cont, fr, workspace, lay, st);
        if (e != hipSuccess) return hip_status(e);
      }
      e = launch_ie_merge(o, lse, 1, T, Hq, d, workspace, lay, st);
    } else {
      e = launch_prefill_f32(mode == JL_MODE_PLAIN ? PASS_PLAIN : PASS_FUSED, xq, v, o, lse, T, B,
                             Hq, Hkv, d, w0, sc, cont, fr, workspace, lay, st);
    }
  }
  if (e == hipSuccess && ev_end) e = hipEventRecord((hipEvent_t)ev_end, st);
  return hip_status(e);
}

int jl_bifocal_prefill(const void* xq, const void* xk, const void* v, void* o, float* lse,
                       void* kcache_out, const int32_t* cu_seqlens, int B, int64_t T, int Hq,
                       int Hkv, int d, int64_t w0, int64_t w_pre, double theta, float scale,
                       jl_dtype dt, jl_mode mode, void* workspace, size_t ws_bytes,
                       void* stream) {
  return jl_bifocal_prefill_timed(xq, xk, v, o, lse, kcache_out, cu_seqlens, B, T, Hq, Hkv, d, w0,
                                  w_pre, theta, scale, dt, mode, workspace, ws_bytes, stream,
                                  nullptr, nullptr);
}

int jl_prefill_flags(const void* workspace, uint32_t* flags, void* stream) {
  if (!workspace || !flags) return JL_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, (const char*)workspace + kHdrFlags * sizeof(int),
                                sizeof(v), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_status(e);
  *flags = v;
  return JL_OK;
}

// ---- prefill continued on an existing absolute cache
static bool cached_shape_ok(int64_t q_off, int64_t Tq, int Hq, int Hkv) {
  if (q_off < 0 || Tq < 0 || !heads_ok(Hq, Hkv)) return false;
  const int64_t lim = (int64_t)INT32_MAX / 2;
  return q_off <= lim && Tq <= lim - q_off;
}

size_t jl_prefill_cached_workspace_size(int64_t q_off, int64_t Tq, int Hq, int Hkv, int d,
                                        jl_mode mode) {
  mode = strip_remap(mode, nullptr);
  if (!cached_shape_ok(q_off, Tq, Hq, Hkv) || d != PF_D) return 0;
  if (mode != JL_MODE_FUSED && mode != JL_MODE_PLAIN) return 0;
  return prefill_layout(q_off + Tq, 1, Hq, Hkv, d, JL_BF16, mode).total;
}

int jl_bifocal_prefill_cached_timed(const void* xq, const void* kcache, const void* vcache,
                                    void* o, float* lse, int64_t q_off, int64_t Tq,
                                    int64_t capacity, int Hq, int Hkv, int d, int64_t w0,
                                    int64_t w_pre, double theta, float scale, jl_dtype dt,
                                    jl_mode mode, void* workspace, size_t ws_bytes, void* stream,
                                    void* ev_begin, void* ev_end) {
  int cont;
  mode = strip_remap(mode, &cont);
  if (!cached_shape_ok(q_off, Tq, Hq, Hkv)) return JL_EINVAL;
  if (capacity < 1 || q_off + Tq > capacity) return JL_EINVAL;
  if (w0 < 0 || w_pre < 1 || !(theta > 1.0) || !(scale == scale)) return JL_EINVAL;
  if (dt != JL_BF16 && dt != JL_FP32) return JL_EINVAL;
  if (mode == JL_MODE_IE) return JL_EUNSUPPORTED;
  if (mode != JL_MODE_FUSED && mode != JL_MODE_PLAIN) return JL_EINVAL;
  if (dt != JL_BF16 || d != PF_D) return JL_EUNSUPPORTED;
  if (w0 > (int64_t)INT32_MAX) w0 = INT32_MAX;
  if (Tq == 0) return JL_OK;
  if (!xq || !kcache || !vcache || !o) return JL_EINVAL;
  const int64_t L = q_off + Tq;
  const PrefillLayout lay = prefill_layout(L, 1, Hq, Hkv, d, dt, mode);
  if (!workspace || ws_bytes < lay.total) return JL_EWORKSPACE;
  if (((uintptr_t)workspace) & 255) return JL_EINVAL;
  const float sc = scale > 0.f ? scale : (float)(1.0 / sqrt((double)d));
  RopeFreqs fr;
  make_freqs(fr, d, theta);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_prefill_plan(nullptr, 1, L, q_off, w_pre, PF_BM, workspace, lay, st);
  if (e != hipSuccess) return hip_status(e);
  e = launch_prefill_prep_bf16(kcache, vcache, nullptr, L, 1, Hkv, mode != JL_MODE_PLAIN, 1,
                               sc * 1.4426950408889634f, cont, fr, workspace, lay, st);
  if (e != hipSuccess) return hip_status(e);
  if (ev_begin && (e = hipEventRecord((hipEvent_t)ev_begin, st)) != hipSuccess)
    return hip_status(e);
  e = launch_prefill_bf16(mode == JL_MODE_PLAIN ? PASS_PLAIN : PASS_FUSED, xq, o, lse, Tq, 1, Hq,
                          Hkv, w0, q_off, sc, cont, fr, workspace, lay, st);
  if (e == hipSuccess && ev_end) e = hipEventRecord((hipEvent_t)ev_end, st);
  return hip_status(e);
}

int jl_bifocal_prefill_cached(const void* xq, const void* kcache, const void* vcache, void* o,
                              float* lse, int64_t q_off, int64_t Tq, int64_t capacity, int Hq,
                              int Hkv, int d, int64_t w0, int64_t w_pre, double theta, float scale,
                              jl_dtype dt, jl_mode mode, void* workspace, size_t ws_bytes,
                              void* stream) {
  return jl_bifocal_prefill_cached_timed(xq, kcache, vcache, o, lse, q_off, Tq, capacity, Hq, Hkv,
                                         d, w0, w_pre, theta, scale, dt, mode, workspace, ws_bytes,
                                         stream, nullptr, nullptr);
}

// bf16 decode: keys per split. One wave per split, four KV heads per
// workgroup, two workgroups fit a CU: aim at a split count that covers the 256
// CUs evenly (two workgroups per CU when each split gets >= 256 keys, else
// one), since a few CUs holding an extra workgroup would set the kernel's
// time. The kernel walks 32-key chunks, so a split of 32 c + 1 keys costs a
// whole extra chunk: sizes are whole chunks, rounded down when that leaves
// only a small last split (its workgroups finish almost at once), else up.
static int64_t decode_bf16_kps(int64_t keys, int Hkv) {
  const int64_t hg = (Hkv + 3) / 4;
  const int64_t s_full = 512 / hg > 0 ? 512 / hg : 1, s_half = 256 / hg > 0 ? 256 / hg : 1;
  int64_t want;
  if (keys >= 256 * s_full) want = s_full;
  else if (keys >= 128 * s_half) want = s_half;
  else want = (keys + 127) / 128;
  const int64_t kc = 32 * ((keys + 32 * want - 1) / (32 * want));
  const int64_t kf = 32 * (keys / (32 * want));
  if (kf >= 32) {
    const int64_t sf = (keys + kf - 1) / kf;
    if (sf == want + 1 && keys - (sf - 1) * kf <= kf / 4) return kf;
  }
  return kc;
}

static int decode_max_splits(int64_t capacity) {
  int64_t s = (capacity + 63) / 64;
  return (int)(s < 1024 ? s : 1024);
}

size_t jl_decode_workspace_size(int64_t capacity, int Hq, int d) {
  if (capacity < 1 || capacity > (int64_t)INT32_MAX || Hq < 1 || Hq > kMaxHeads || !dim_ok(d))
    return 0;
  return align256((size_t)Hq * decode_max_splits(capacity) * (d + 2) * sizeof(float));
}

int jl_bifocal_decode_timed(const void* xq, const void* kcache, const void* vcache, void* o,
                            float* lse, int64_t pos, int64_t capacity, int Hq, int Hkv, int d,
                            int64_t w0, int64_t w_pre, double theta, float scale, jl_dtype dt,
                            jl_mode mode, int num_splits, void* workspace, size_t ws_bytes,
                            void* stream, void* ev_begin, void* ev_end) {
  int cont;
  mode = strip_remap(mode, &cont);
  if (pos < 0 || capacity < 1 || pos >= capacity || capacity > (int64_t)INT32_MAX) return JL_EINVAL;
  if (!heads_ok(Hq, Hkv) || w0 < 0 || w_pre < 1 || !(theta > 1.0)) return JL_EINVAL;
  if (num_splits < 0 || !(scale == scale)) return JL_EINVAL;
  if (dt != JL_BF16 && dt != JL_FP32) return JL_EINVAL;
  if (mode == JL_MODE_IE) return JL_EUNSUPPORTED;
  if (mode != JL_MODE_FUSED && mode != JL_MODE_PLAIN) return JL_EINVAL;
  if (d != 128 && d != 64) return JL_EUNSUPPORTED;
  {
    const int r = Hq / Hkv;
    if (r != 1 && r != 2 && r != 4 && r != 8) return JL_EUNSUPPORTED;
  }
  if (!xq || !kcache || !vcache || !o) return JL_EINVAL;
  const int maxs = decode_max_splits(capacity);
  const int64_t keys = pos + 1;
  if (num_splits > maxs) return JL_EINVAL;
  int64_t kps;
  if (num_splits == 0 && dt == JL_BF16) {
    kps = decode_bf16_kps(keys, Hkv);
  } else {
    int64_t S0 = num_splits;
    if (S0 == 0) {
      // float32: one workgroup per split, ~4 per CU, at least 64 keys
      const int64_t want = (1024 + Hkv - 1) / Hkv, by_keys = (keys + 63) / 64;
      S0 = want < by_keys ? want : by_keys;
    }
    if (S0 > keys) S0 = keys;
    kps = (keys + S0 - 1) / S0;
  }
  if ((keys + kps - 1) / kps > maxs) kps = (keys + maxs - 1) / maxs;
  const int S = (int)((keys + kps - 1) / kps);  // no empty split
  const size_t need = (size_t)Hq * S * (d + 2) * sizeof(float);
  if (!workspace || ws_bytes < need) return JL_EWORKSPACE;
  if (((uintptr_t)workspace) & 15) return JL_EINVAL;
  const float sc = scale > 0.f ? scale : (float)(1.0 / sqrt((double)d));
  RopeFreqs fr;
  make_freqs(fr, d, theta);
  const int64_t G = jl::group_size(pos + 1, w_pre);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (ev_begin && (e = hipEventRecord((hipEvent_t)ev_begin, st)) != hipSuccess)
    return hip_status(e);
  e = launch_decode(xq, kcache, vcache, o, lse, pos, Hq, Hkv, d,
                    w0 > (int64_t)INT32_MAX ? INT32_MAX : w0, G, sc, fr, mode == JL_MODE_PLAIN,
                    cont, dt == JL_FP32, (int)kps, workspace, st);
  if (e == hipSuccess && ev_end) e = hipEventRecord((hipEvent_t)ev_end, st);
  return hip_status(e);
}

// ---- batched decode
// fp32: one workgroup per (split, KV head, sequence), ~4 per CU in all
static int decode_batch_f32_splits(int B, int64_t max_keys, int Hkv) {
  const int64_t units = (int64_t)B * Hkv;
  const int64_t by_wg = 1024 / units > 0 ? 1024 / units : 1;
  const int64_t by_keys = (max_keys + 63) / 64;
  const int64_t want = by_wg < by_keys ? by_wg : by_keys;
  return want < 1 ? 1 : (int)want;
}

// Partials [B, Hq, S, d + 2] fp32, then the bf16 work list int32 [B + 1].
static size_t decode_batch_list_offset(int B, int Hq, int S, int d) {
  return align256((size_t)B * Hq * S * (d + 2) * sizeof(float));
}

size_t jl_decode_batch_workspace_size(int B, int64_t max_keys, int Hq, int d) {
  if (B < 1 || B > 65535 || max_keys < 1 || max_keys > (int64_t)INT32_MAX || Hq < 1 ||
      Hq > kMaxHeads || !dim_ok(d))
    return 0;
  return decode_batch_list_offset(B, Hq, decode_max_splits(max_keys), d) +
         align256((size_t)(B + 1) * sizeof(int));
}

int jl_bifocal_decode_batch_timed(const void* xq, const void* kcache, const void* vcache, void* o,
                                  float* lse, const int32_t* positions,
                                  const int32_t* cache_starts, int B, int64_t max_keys,
                                  int64_t cache_rows, int Hq, int Hkv, int d, int64_t w0,
                                  int64_t w_pre, double theta, float scale, jl_dtype dt,
                                  jl_mode mode, int num_splits, void* workspace, size_t ws_bytes,
                                  void* stream, void* ev_begin, void* ev_end) {
  int cont;
  mode = strip_remap(mode, &cont);
  if (B < 0 || B > 65535 || max_keys < 1 || max_keys > (int64_t)INT32_MAX || cache_rows < 1)
    return JL_EINVAL;
  if (!heads_ok(Hq, Hkv) || w0 < 0 || w_pre < 1 || !(theta > 1.0)) return JL_EINVAL;
  if (num_splits < 0 || !(scale == scale)) return JL_EINVAL;
  if (dt != JL_BF16 && dt != JL_FP32) return JL_EINVAL;
  if (mode == JL_MODE_IE) return JL_EUNSUPPORTED;
  if (mode != JL_MODE_FUSED && mode != JL_MODE_PLAIN) return JL_EINVAL;
  if (d != 128 && d != 64) return JL_EUNSUPPORTED;
  {
    const int r = Hq / Hkv;
    if (r != 1 && r != 2 && r != 4 && r != 8) return JL_EUNSUPPORTED;
  }
  if (B == 0) return JL_OK;
  if (!xq || !kcache || !vcache || !o || !positions || !cache_starts) return JL_EINVAL;
  const int maxs = decode_max_splits(max_keys);
  // bf16: the splits of the longest sequence are sized as a single decode of
  // it would size them; every sequence is cut into splits of that many keys
  // and a fixed grid walks the resulting work list. fp32: one grid over all
  // (split, head, sequence) triples.
  if (num_splits > maxs) return JL_EINVAL;
  int64_t kps;
  if (num_splits == 0 && dt == JL_BF16) {
    kps = decode_bf16_kps(max_keys, Hkv);
  } else {
    int64_t S0 = num_splits ? num_splits : decode_batch_f32_splits(B, max_keys, Hkv);
    if (S0 > max_keys) S0 = max_keys;
    kps = (max_keys + S0 - 1) / S0;
  }
  if ((max_keys + kps - 1) / kps > maxs) kps = (max_keys + maxs - 1) / maxs;
  const int S = (int)((max_keys + kps - 1) / kps);  // no split past max_keys
  const size_t list_off = decode_batch_list_offset(B, Hq, S, d);
  const size_t need = list_off + (size_t)(B + 1) * sizeof(int);
  if (!workspace || ws_bytes < need) return JL_EWORKSPACE;
  const int64_t hg = (Hkv + 3) / 4;
  const int64_t units = (int64_t)B * S * hg;  // upper bound of the work list
  const int grid_wg = (int)(units < 512 ? units : 512);  // two workgroups per CU
  if (((uintptr_t)workspace) & 15) return JL_EINVAL;
  const float sc = scale > 0.f ? scale : (float)(1.0 / sqrt((double)d));
  RopeFreqs fr;
  make_freqs(fr, d, theta);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (ev_begin && (e = hipEventRecord((hipEvent_t)ev_begin, st)) != hipSuccess)
    return hip_status(e);
  e = launch_decode_batch(xq, kcache, vcache, o, lse, positions, cache_starts, B, max_keys,
                          cache_rows, Hq, Hkv, d, w0 > (int64_t)INT32_MAX ? INT32_MAX : w0,
                          w_pre > (int64_t)INT32_MAX ? (int64_t)INT32_MAX : w_pre, sc, fr,
                          mode == JL_MODE_PLAIN, cont, dt == JL_FP32, S, (int)kps, workspace,
                          (int*)((char*)workspace + list_off), grid_wg, st);
  if (e == hipSuccess && ev_end) e = hipEventRecord((hipEvent_t)ev_end, st);
  return hip_status(e);
}

int jl_bifocal_decode_batch(const void* xq, const void* kcache, const void* vcache, void* o,
                            float* lse, const int32_t* positions, const int32_t* cache_starts,
                            int B, int64_t max_keys, int64_t cache_rows, int Hq, int Hkv, int d,
                            int64_t w0, int64_t w_pre, double theta, float scale, jl_dtype dt,
                            jl_mode mode, int num_splits, void* workspace, size_t ws_bytes,
                            void* stream) {
  return jl_bifocal_decode_batch_timed(xq, kcache, vcache, o, lse, positions, cache_starts, B,
                                       max_keys, cache_rows, Hq, Hkv, d, w0, w_pre, theta, scale,
                                       dt, mode, num_splits, workspace, ws_bytes, stream, nullptr,
                                       nullptr);
}

int jl_bifocal_decode(const void* xq, const void* kcache, const void* vcache, void* o, float* lse,
                      int64_t pos, int64_t capacity, int Hq, int Hkv, int d, int64_t w0,
                      int64_t w_pre, double theta, float scale, jl_dtype dt, jl_mode mode,
                      int num_splits, void* workspace, size_t ws_bytes, void* stream) {
  return jl_bifocal_decode_timed(xq, kcache, vcache, o, lse, pos, capacity, Hq, Hkv, d, w0, w_pre,
                                 theta, scale, dt, mode, num_splits, workspace, ws_bytes, stream,
                                 nullptr, nullptr);
}

}  // extern "C"

// ---- decode without allocation, for callers that cannot allocate
// The partials live in a file-scope device array instead of a caller
// workspace. Its name is a host-side stand-in in host code: the device
// address is looked up once per device (hipGetSymbolAddress with that device
// current) and only that address is passed to the kernels.
static __device__ __attribute__((aligned(256))) uint8_t scratch[JL_NOALLOC_SCRATCH_BYTES];
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];  // per device ordinal

static int scratch_pointer(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= 64) return JL_EINVAL;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return JL_OK;
}

extern "C" {

int jl_bifocal_decode_noalloc(const void* xq, const void* kcache, const void* vcache, void* o,
                              float* lse, int64_t pos, int64_t capacity, int Hq, int Hkv, int d,
                              int64_t w0, int64_t w_pre, double theta, float scale, jl_dtype dt,
                              jl_mode mode, int num_splits, void* stream) {
  void* ws = nullptr;
  const int st = scratch_pointer(&ws);
  if (st != JL_OK) return st;
  // the same checks, split plan and kernels as jl_bifocal_decode; a plan whose
  // partials exceed the array comes back as JL_EWORKSPACE before any launch
  return jl_bifocal_decode_timed(xq, kcache, vcache, o, lse, pos, capacity, Hq, Hkv, d, w0, w_pre,
                                 theta, scale, dt, mode, num_splits, ws, JL_NOALLOC_SCRATCH_BYTES,
                                 stream, nullptr, nullptr);
}

int jl_debug_tile_classes(int64_t L, int64_t w0, int8_t* out_dev, void* stream) {
  if (L < 1 || L > (int64_t)1 << 24 || w0 < 0 || !out_dev) return JL_EINVAL;
  return hip_status(launch_tile_dump(L, w0, out_dev, (hipStream_t)stream));
}

int jl_calib_stream_read_ex(const void* src, size_t bytes, uint32_t* sink, int blocks,
                            int variant, void* stream) {
  if (!src || !sink || bytes < 16 || (bytes & 15) || (((uintptr_t)src) & 15) || blocks < 1)
    return JL_EINVAL;
  if (variant < 0 || variant > 4) return JL_EINVAL;
  return hip_status(launch_calib_read(src, bytes, sink, blocks, variant, (hipStream_t)stream));
}

int jl_calib_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks,
                         void* stream) {
  return jl_calib_stream_read_ex(src, bytes, sink, blocks, 0, stream);
}

int jl_calib_mfma_bf16(float* sink, int blocks, int iters, void* stream) {
  if (!sink || blocks < 1 || iters < 1) return JL_EINVAL;
  return hip_status(launch_calib_mfma(sink, blocks, iters, (hipStream_t)stream));
}

const char* jl_status_string(int status) {
  switch (status) {
    case JL_OK: return "ok";
    case JL_EINVAL: return "invalid argument";
    case JL_EUNSUPPORTED: return "unsupported head dim, dtype or mode";
    case JL_EHIP: return "HIP runtime or launch error";
    case JL_EWORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int jl_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
