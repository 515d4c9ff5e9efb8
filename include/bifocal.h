/*
 * libbifocal -- dynamic bifocal RoPE attention on AMD Instinct MI355X (gfx950).
 *
 * The method (Jet-Long, "Efficient Long-Context Extension with Dynamic
 * Bifocal RoPE"): causal softmax attention whose score for query position q
 * and key position k is
 *     RoPE(x_q, q)    . RoPE(x_k, k)       when q - k <= w0   (local window)
 *     RoPE(x_q, f(q)) . RoPE(x_k, f(k))    when q - k >  w0   (remote view)
 * with f(x) = floor(x / G) and G = max(1, ceil(L / w_pretrained)).
 *   - r9-hu paper digest of the paper, section Method: Eq. 1 (the score), the
 *     "Dynamic group size" paragraph (G, f), the "KV cache invariant"
 *     paragraph (absolute keys in the cache, correction offsets
 *     Delta = f(x) - x, R_a R_b = R_{a+b}) and the "Inclusion-exclusion
 *     prefill" paragraph (three passes merged by LSE weights).
 *   - pith.science review of arXiv 2607.07740, axiom ledger: Sec. 3.1 Eq. 2,
 *     Sec. 3.2 Eqs. 5-6, Sec. 3.3 Eq. 7.
 *
 * Conventions shared by every entry point:
 *   - Positions are 0-based and restart at each sequence's first token.
 *   - RoPE rotates the pair (x_i, x_{i+d/2}) by p * theta^(-2i/d),
 *     i = 0 .. d/2-1 (rotate-half pairing). Angles are formed and reduced
 *     modulo 2*pi in float64 before float32 sin/cos.
 *   - q - k == w0 is local. The softmax scale defaults to 1/sqrt(d).
 *   - GQA: query head h reads KV head h / (Hq / Hkv).
 *   - Token-major packed layouts: [T, H, d] row-major, d contiguous, every
 *     base pointer 16-byte aligned. LSE is [Hq, T] float32, natural log.
 *   - "void* stream" is a hipStream_t (NULL = the default stream). All device
 *     work is asynchronous on that stream; the caller owns every buffer.
 *   - The library never allocates device memory, keeps no state between
 *     calls and never writes the inputs (the KV cache included).
 *   - Errors: arguments are validated on the host BEFORE any launch; a
 *     failing check returns a negative status and launches nothing. A HIP
 *     launch failure returns JL_EHIP (see jl_last_hip_error()). Faults that
 *     happen later on the device surface at the caller's synchronisation.
 *     No entry point aborts or prints.
 */
#ifndef BIFOCAL_H
#define BIFOCAL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define JL_OK 0
#define JL_EINVAL (-1)       /* bad scalar, shape or pointer argument            */
#define JL_EUNSUPPORTED (-2) /* head dim / dtype / mode combination not built    */
#define JL_EHIP (-3)         /* HIP launch or runtime error                      */
#define JL_EWORKSPACE (-4)   /* workspace NULL or smaller than the size query    */

/* The enums are int-sized in both languages; in C++ they get int as their
 * fixed underlying type, so any int a C caller passes (an unsupported dtype,
 * a mode with flags OR-ed in) is a valid value there too and is rejected or
 * decoded by the callee, never undefined. */
#ifdef __cplusplus
#define JL_ENUM_BASE : int
#else
#define JL_ENUM_BASE
#endif

typedef enum JL_ENUM_BASE { JL_BF16 = 0, JL_FP32 = 1 } jl_dtype;

/* FUSED: one pass, each (query tile, key tile) classified local / remote /
 *        boundary, per-element select on boundary tiles.
 * IE:    the pages' three attention passes (window+absolute, causal+remapped,
 *        window+remapped) merged by Eq. 7. A checked alternative, NOT exact
 *        in floating point: Eq. 7 subtracts pass C's weighted output from
 *        pass B's, and on a row whose cancellation ratio (stored at
 *        jl_prefill_ie_ratio_offset) is large the float32 passes lose digits
 *        in proportion; above a ratio of about 1e3 the row's output is
 *        unreliable (on peaked 128K inputs about 1% of rows, errors up to
 *        1e5). FUSED has no subtraction and meets the tolerance on every row.
 * PLAIN: ordinary causal RoPE attention (every pair local) -- the baseline
 *        the bifocal overhead is measured against. */
typedef enum JL_ENUM_BASE { JL_MODE_FUSED = 0, JL_MODE_IE = 1, JL_MODE_PLAIN = 2 } jl_mode;

/* Remote-map flag, OR-ed into the mode argument of every call that takes one
 * (e.g. (jl_mode)(JL_MODE_FUSED | JL_REMAP_CONTINUOUS)). Without it the
 * remote branch of Eq. 1 rotates at f(x) = floor(x / G), the aliasing map.
 * With it f(x) = x / G as a real number: continuous frequency interpolation by
 * the same G, the arm the aliasing map is compared against in the pith.science
 * review's Table 6 discussion (Referee Report major comment 2; ledger axiom on
 * the discrete angle grid). The window, G, routing and tiling are unchanged,
 * and the cached keys are corrected by the real-angle rotation R_{k/G - k}.
 * JL_MODE_PLAIN has no remote pair and ignores the flag. */
#define JL_REMAP_CONTINUOUS 16

/* Eq. 2: G = max(1, ceil(L / w_pre)) in exact integer arithmetic.
 * Returns G >= 1, or JL_EINVAL when L < 1 or w_pre < 1. Host only. */
int64_t jl_group_size(int64_t L, int64_t w_pre);

/* Class of the tile with query positions q0..q1 and key positions k0..k1
 * (inclusive, sequence-relative), from the routing condition of Eq. 1:
 *   0 masked   (k0 > q1: no causal pair)
 *   1 local    (q1 - k0 <= w0: every causal pair is in the window)
 *   2 remote   (q0 - k1 >  w0: every causal pair is outside it)
 *   3 boundary (both kinds)
 *   +4 when the causal diagonal crosses the tile (k1 > q0), for classes 1/3.
 * Depends on distances only, never on G. JL_EINVAL if q0 > q1, k0 > k1, any
 * position is negative, or w0 < 0. Host only. */
int jl_tile_class(int64_t q0, int64_t q1, int64_t k0, int64_t k1, int64_t w0);

/* Query-tile rows (BM) and key-tile width (BN) the prefill kernels use for
 * dtype dt and head dim d. JL_EUNSUPPORTED if that combination is not built. */
int jl_prefill_tile_shape(jl_dtype dt, int d, int* bm, int* bn);

/* Absolute RoPE in place: x[t, h, :] = RoPE(x[t, h, :], pos(t)) where
 * pos(t) = pos_offset + (t - start of t's sequence). x: [T, H, d] bf16 or
 * fp32 on the device. cu_seqlens: device int32 [B+1] prefix offsets
 * (cu_seqlens[0] = 0, cu_seqlens[B] = T), or NULL for one sequence (B is then
 * ignored). This is how keys enter the absolute KV cache ("KV cache
 * invariant" paragraph of the digest's Method section).
 * Errors: JL_EINVAL (NULL x, T < 0, H < 1, d odd or > 256, pos_offset < 0,
 * theta <= 1, B < 1 with cu_seqlens), JL_EUNSUPPORTED (d not a multiple of
 * 16), JL_EHIP. T == 0 is a no-op. */
int jl_rope_apply(void* x, int64_t T, int H, int d, const int32_t* cu_seqlens, int B,
                  int64_t pos_offset, double theta, jl_dtype dt, void* stream);

/* Bytes of device workspace jl_bifocal_prefill needs for these sizes. */
size_t jl_prefill_workspace_size(int64_t T, int B, int Hq, int Hkv, int d, jl_dtype dt,
                                 jl_mode mode);

/* Byte offset, inside a prefill workspace sized for these arguments, of the
 * float32 [Hq, T] array where JL_MODE_IE stores each row's cancellation ratio
 * (W_B + W_C) / (W_A + W_B - W_C) of Eq. 7: how much the subtraction of
 * pass C can amplify rounding in that row (small values are benign). */
size_t jl_prefill_ie_ratio_offset(int64_t T, int B, int Hq, int Hkv, int d, jl_dtype dt);

/* Range flags a bf16 prefill leaves in its workspace (read them with
 * jl_prefill_flags). The QK^T operands are fp16: a rotated query, or a key
 * times the score scale times log2(e), outside the fp16 range (|x| > 65504)
 * becomes infinite and the affected rows come out NaN or wrong. The kernels
 * detect it and set a bit; they neither stop nor fault. NaN inputs also set
 * the bit of the operand they reach. */
#define JL_FLAG_Q_RANGE 1 /* a rotated query operand was not a finite fp16 value */
#define JL_FLAG_K_RANGE 2 /* a scaled key operand was not a finite fp16 value    */

/* Reads the range flags (JL_FLAG_*) of the last jl_bifocal_prefill or
 * jl_bifocal_prefill_cached call that used `workspace` (device memory) into
 * *flags (host). Waits for `stream` to finish first, so call it on the stream
 * of the prefill. Every bf16 prefill call clears the flags before its kernels
 * run; fp32 calls (no 16-bit operands) leave them 0. Errors: JL_EINVAL (NULL
 * pointer), JL_EHIP. */
int jl_prefill_flags(const void* workspace, uint32_t* flags, void* stream);

/* Causal bifocal attention over a packed batch (Eq. 1; Eq. 7 in IE mode).
 *   xq  [T, Hq, d]  RAW (not yet rotated) queries      bf16 | fp32
 *   xk  [T, Hkv, d] RAW keys                            bf16 | fp32
 *   v   [T, Hkv, d] values                              bf16 | fp32
 *   o   [T, Hq, d]  output (overwritten)                bf16 | fp32
 *   lse [Hq, T]     float32 natural-log LSE per row, or NULL
 *   kcache_out [T, Hkv, d] or NULL: receives RoPE(xk, absolute position),
 *       the same values jl_rope_apply writes, so one call also fills the
 *       absolute KV cache for later decoding.
 *   cu_seqlens: device int32 [B+1] (as in jl_rope_apply) or NULL for one
 *       sequence of length T (B must then be 1). Every sequence takes its own
 *       G from its own length.
 *   w0 >= 0, w_pre >= 1, theta > 1, scale <= 0 selects 1/sqrt(d).
 * The kernels rotate the raw vectors directly to the absolute and the
 * remapped positions (the correction rotation of the cached keys by
 * R_{f(k)-k} gives the same vectors by R_a R_b = R_{a+b}; starting from the
 * raw inputs avoids rounding the absolute vectors twice).
 * Supported: bf16 with d = 128 (all modes); fp32 with d = 64 or 128.
 * Range (bf16): the QK^T operands are fp16, the keys carrying the score scale
 * times log2(e), so rotated queries must stay below 65504 in magnitude and
 * keys below 65504 / (scale log2 e) (about 5.1e5 at d = 128); beyond that the
 * scores overflow, the outputs of the affected rows are undefined (NaN or
 * wrong) and the call sets JL_FLAG_Q_RANGE / JL_FLAG_K_RANGE in the workspace
 * (jl_prefill_flags); the status returned is still JL_OK. Values: the fp32
 * softmax sums stay finite while max |v| * 2^65 * (key tiles of 64) < 2^128,
 * i.e. |v| < 2^50 at 128K keys.
 * Workspace: jl_prefill_workspace_size(...) bytes of device memory, any
 * contents, 256-byte aligned; it holds the rotated key tiles, the transposed
 * values and the tile schedule. Errors: JL_EINVAL, JL_EUNSUPPORTED,
 * JL_EWORKSPACE, JL_EHIP. T == 0 is a no-op. */
int jl_bifocal_prefill(const void* xq, const void* xk, const void* v, void* o, float* lse,
                       void* kcache_out, const int32_t* cu_seqlens, int B, int64_t T, int Hq,
                       int Hkv, int d, int64_t w0, int64_t w_pre, double theta, float scale,
                       jl_dtype dt, jl_mode mode, void* workspace, size_t ws_bytes, void* stream);

/* jl_bifocal_prefill plus timing: ev_begin / ev_end (hipEvent_t created by the
 * caller, or NULL) are recorded on `stream` immediately before the first and
 * after the last attention kernel (FUSED / PLAIN: the attention pass; IE: the
 * three passes and the Eq. 7 merge), excluding the schedule and the key/value
 * pre-pass, so a caller can time the dominant kernel alone. Same arguments,
 * errors and results as jl_bifocal_prefill; no events are recorded when the
 * call returns an error before launching. */
int jl_bifocal_prefill_timed(const void* xq, const void* xk, const void* v, void* o, float* lse,
                             void* kcache_out, const int32_t* cu_seqlens, int B, int64_t T,
                             int Hq, int Hkv, int d, int64_t w0, int64_t w_pre, double theta,
                             float scale, jl_dtype dt, jl_mode mode, void* workspace,
                             size_t ws_bytes, void* stream, void* ev_begin, void* ev_end);

/* Bytes of device workspace jl_bifocal_prefill_cached needs for a chunk of
 * Tq query rows starting at position q_off (mode FUSED or PLAIN, d = 128);
 * 0 for arguments it would reject. */
size_t jl_prefill_cached_workspace_size(int64_t q_off, int64_t Tq, int Hq, int Hkv, int d,
                                        jl_mode mode);

/* Prefill continued on an existing absolute cache (chunked prefill): the
 * Tq query rows at positions q_off .. q_off + Tq - 1 of one sequence attend
 * causally to keys 0 .. q_off + Tq - 1 held in the cache, with
 * L = q_off + Tq and G = max(1, ceil(L / w_pre)) (Eq. 1 with the "Dynamic
 * group size" of the whole sequence so far). The cache keeps keys rotated at
 * their absolute positions, so a chunk that moves L across a multiple of
 * w_pre (G changes) needs no re-rotation of the cache: remote keys get
 * R_{f(k) - k} on the fly ("KV cache invariant" paragraph; Pith ledger
 * Sec. 3.2 Eqs. 5-6).
 *   xq      [Tq, Hq, d]        RAW queries of the chunk (bf16)
 *   kcache  [capacity, Hkv, d] keys rotated at absolute positions, rows
 *                              0 .. q_off + Tq - 1 filled (the chunk's own
 *                              keys included, e.g. written by jl_rope_apply
 *                              with pos_offset = q_off); never written
 *   vcache  [capacity, Hkv, d] values, same rows; never written
 *   o       [Tq, Hq, d] bf16; lse [Hq, Tq] float32 (natural log) or NULL.
 * q_off = 0 is an ordinary single-sequence prefill from the cache; Tq = 1
 * is one decode step. Supported: bf16, d = 128, JL_MODE_FUSED or
 * JL_MODE_PLAIN (JL_MODE_IE: JL_EUNSUPPORTED). Errors: JL_EINVAL (q_off < 0,
 * Tq < 0, q_off + Tq > capacity, bad heads or scalars, NULL pointers),
 * JL_EUNSUPPORTED, JL_EWORKSPACE, JL_EHIP. Tq = 0 is a no-op. */
int jl_bifocal_prefill_cached(const void* xq, const void* kcache, const void* vcache, void* o,
                              float* lse, int64_t q_off, int64_t Tq, int64_t capacity, int Hq,
                              int Hkv, int d, int64_t w0, int64_t w_pre, double theta, float scale,
                              jl_dtype dt, jl_mode mode, void* workspace, size_t ws_bytes,
                              void* stream);

/* jl_bifocal_prefill_cached plus timing: ev_begin / ev_end (caller-created
 * hipEvent_t, or NULL) bracket the attention kernel on `stream`. */
int jl_bifocal_prefill_cached_timed(const void* xq, const void* kcache, const void* vcache,
                                    void* o, float* lse, int64_t q_off, int64_t Tq,
                                    int64_t capacity, int Hq, int Hkv, int d, int64_t w0,
                                    int64_t w_pre, double theta, float scale, jl_dtype dt,
                                    jl_mode mode, void* workspace, size_t ws_bytes, void* stream,
                                    void* ev_begin, void* ev_end);

/* Bytes of device workspace jl_bifocal_decode needs (for any pos < capacity
 * and any num_splits it would choose or accept). */
size_t jl_decode_workspace_size(int64_t capacity, int Hq, int d);


/* One generation step at position pos (0-based) against the absolute cache:
 * L = pos + 1 and G = max(1, ceil(L / w_pre)); keys 0..pos are read, the
 * cache is never written ("KV cache invariant" paragraph; Pith ledger
 * Sec. 3.2 Eqs. 5-6).
 *   xq      [Hq, d]            RAW query of the token at pos   bf16 | fp32
 *   kcache  [capacity, Hkv, d] keys already rotated at their absolute
 *                              positions (jl_rope_apply / kcache_out)
 *   vcache  [capacity, Hkv, d] values
 *   o       [Hq, d] output; lse [Hq] float32 or NULL.
 * Remote keys (pos - k > w0) are corrected on the fly by R_{f(k) - k} and
 * scored against RoPE(xq, f(pos)); local keys are scored against
 * RoPE(xq, pos). JL_MODE_PLAIN scores every key as local (the baseline);
 * JL_MODE_IE is not a decode mode (JL_EUNSUPPORTED).
 * num_splits: key-range splits merged by LSE; 0 lets the library choose.
 * Workspace: jl_decode_workspace_size bytes, 16-byte aligned, any contents.
 * Range (bf16): keys and the query times scale log2(e) are fp16 operands; a
 * value beyond 65504 in magnitude (or a NaN) makes the outputs and LSE of
 * the query heads of that key's KV head NaN. Nothing faults and the status
 * is still JL_OK.
 * Supported: bf16 or fp32, d = 128 or 64, Hq / Hkv in {1, 2, 4, 8}.
 * Errors: JL_EINVAL (pos < 0, pos >= capacity, bad heads, NULL pointers,
 * num_splits < 0), JL_EUNSUPPORTED, JL_EWORKSPACE, JL_EHIP. */
int jl_bifocal_decode(const void* xq, const void* kcache, const void* vcache, void* o, float* lse,
                      int64_t pos, int64_t capacity, int Hq, int Hkv, int d, int64_t w0,
                      int64_t w_pre, double theta, float scale, jl_dtype dt, jl_mode mode,
                      int num_splits, void* workspace, size_t ws_bytes, void* stream);

/* jl_bifocal_decode plus timing: ev_begin / ev_end (caller-created hipEvent_t,
 * or NULL) bracket the split and merge kernels on `stream`. */
int jl_bifocal_decode_timed(const void* xq, const void* kcache, const void* vcache, void* o,
                            float* lse, int64_t pos, int64_t capacity, int Hq, int Hkv, int d,
                            int64_t w0, int64_t w_pre, double theta, float scale, jl_dtype dt,
                            jl_mode mode, int num_splits, void* workspace, size_t ws_bytes,
                            void* stream, void* ev_begin, void* ev_end);

/* jl_bifocal_decode for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid it): the
 * same arguments without a workspace, the same kernels and results. The split
 * partials live in one file-scope device array of JL_NOALLOC_SCRATCH_BYTES
 * per GPU, held from the library's load until the process ends; its device
 * address is looked up on a device's first call. No entry point allocates.
 * A call whose partials (Hq x splits x (d + 2) floats, after the alignment
 * of jl_decode_workspace_size) would not fit returns JL_EWORKSPACE before
 * any launch. With num_splits = 0 the bf16 split choice fits for Hq <= 32 at
 * d = 128 and any position (it picks at most 512 splits when Hkv <= 4, 256
 * when Hkv <= 8: at most 8.5 MB of partials).
 * Every call on one GPU shares that GPU's array, and nothing in it needs to
 * start at zero: calls that overlap in time on one GPU (other streams, other
 * threads) race and must be serialised by the caller. */
#define JL_NOALLOC_SCRATCH_BYTES (16u << 20)
int jl_bifocal_decode_noalloc(const void* xq, const void* kcache, const void* vcache, void* o,
                              float* lse, int64_t pos, int64_t capacity, int Hq, int Hkv, int d,
                              int64_t w0, int64_t w_pre, double theta, float scale, jl_dtype dt,
                              jl_mode mode, int num_splits, void* stream);

/* Bytes of device workspace jl_bifocal_decode_batch needs for B sequences
 * whose positions are all below max_keys (any num_splits it would choose or
 * accept); 0 for arguments it would reject. */
size_t jl_decode_batch_workspace_size(int B, int64_t max_keys, int Hq, int d);

/* One generation step for each of B independent sequences in one launch
 * (decode as in jl_bifocal_decode, per sequence: L = pos_b + 1 and its own
 * G = max(1, ceil(L / w_pre)), "Dynamic group size" of the digest's Method;
 * remote keys corrected by R_{f(k) - k}, "KV cache invariant"). The caches of
 * the sequences share one buffer of cache_rows rows; sequence b's key k is
 * row cache_starts[b] + k, so packed (varlen) and padded layouts both fit.
 *   xq           [B, Hq, d]         RAW query of each sequence's new token
 *   kcache       [cache_rows, Hkv, d] keys rotated at their absolute positions
 *   vcache       [cache_rows, Hkv, d] values; neither cache is written
 *   o            [B, Hq, d]; lse [B, Hq] float32 (natural log) or NULL
 *   positions    device int32 [B]: pos_b, keys 0 .. pos_b are read
 *   cache_starts device int32 [B]: first cache row of sequence b
 *   max_keys     host bound with pos_b + 1 <= max_keys for every b: the split
 *                plan and the workspace are sized for it
 * The per-sequence values stay on the device (the step can be replayed with
 * new positions without a host round trip). An entry with pos_b < 0,
 * pos_b >= max_keys, cache_starts[b] < 0 or cache_starts[b] + pos_b >=
 * cache_rows reads nothing and gets NaN in o (and lse); the other entries are
 * unaffected. num_splits: splits of max_keys / num_splits keys each, 0 lets the
 * library choose. Workspace: jl_decode_batch_workspace_size bytes, any
 * contents. Range (bf16): as in jl_bifocal_decode, per sequence and KV head.
 * Supported: bf16 or fp32, d = 128 or 64, Hq / Hkv in
 * {1, 2, 4, 8}; mode FUSED or PLAIN, optionally with JL_REMAP_CONTINUOUS.
 * Errors: JL_EINVAL (B < 0 or > 65535, max_keys < 1 or > 2^31 - 1,
 * cache_rows < 1, bad heads or scalars, NULL pointers), JL_EUNSUPPORTED,
 * JL_EWORKSPACE, JL_EHIP. B == 0 is a no-op. */
int jl_bifocal_decode_batch(const void* xq, const void* kcache, const void* vcache, void* o,
                            float* lse, const int32_t* positions, const int32_t* cache_starts,
                            int B, int64_t max_keys, int64_t cache_rows, int Hq, int Hkv, int d,
                            int64_t w0, int64_t w_pre, double theta, float scale, jl_dtype dt,
                            jl_mode mode, int num_splits, void* workspace, size_t ws_bytes,
                            void* stream);

/* jl_bifocal_decode_batch plus timing: ev_begin / ev_end (caller-created
 * hipEvent_t, or NULL) bracket the batch kernels on `stream` (bf16: the work
 * list plan, split and merge kernels; fp32: split and merge kernels). */
int jl_bifocal_decode_batch_timed(const void* xq, const void* kcache, const void* vcache, void* o,
                                  float* lse, const int32_t* positions,
                                  const int32_t* cache_starts, int B, int64_t max_keys,
                                  int64_t cache_rows, int Hq, int Hkv, int d, int64_t w0,
                                  int64_t w_pre, double theta, float scale, jl_dtype dt,
                                  jl_mode mode, int num_splits, void* workspace, size_t ws_bytes,
                                  void* stream, void* ev_begin, void* ev_end);

/* Device-side tile classifier dump: out_dev[i * nk + j] (int8, device) gets
 * the class the prefill kernels compute for query tile i and key tile j of a
 * length-L sequence, nq = ceil(L / BM), nk = ceil(L / BN) with BM, BN from
 * jl_prefill_tile_shape(JL_BF16, 128, ...). For bit-exact checks against
 * jl_tile_class and an independent definition. */
int jl_debug_tile_classes(int64_t L, int64_t w0, int8_t* out_dev, void* stream);

/* Calibration kernels (not part of the method) for the rooflines reported
 * beside the vendor peaks. jl_calib_stream_read reads `bytes` bytes at `src`
 * (device, 16-byte aligned, bytes a multiple of 16) once, with `blocks`
 * workgroups of 256 threads; *sink (device uint32) is left untouched unless
 * the reads xor to one fixed value. jl_calib_mfma_bf16 runs `iters` rounds of
 * four independent 32x32x16 bf16 MFMAs per wave in `blocks` workgroups of 256
 * threads and writes one float per thread to sink (device, blocks * 256
 * floats); one round is 4 * 32768 FLOP per wave. Both only launch on
 * `stream`; time them with the caller's events. JL_EINVAL on bad arguments. */
int jl_calib_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, void* stream);
/* The same streaming read by one of three kernels, so a caller can report the
 * best read rate any of them reaches: variant 0 is jl_calib_stream_read
 * (grid-stride 16-byte loads, four in flight per thread); 1 reads 32 KiB
 * chunks per workgroup with eight nontemporal 16-byte loads in flight per
 * thread; 2 moves 64 KiB chunks by direct global -> LDS transfers (sixteen
 * 1 KiB transfers per wave), the path the bf16 decode streams its values
 * through; 3 is variant 1 without the nontemporal hint and 4 is variant 2
 * with it. Bytes past the last whole chunk are read by ordinary loads.
 * JL_EINVAL on bad arguments or an unknown variant. */
int jl_calib_stream_read_ex(const void* src, size_t bytes, uint32_t* sink, int blocks,
                            int variant, void* stream);
int jl_calib_mfma_bf16(float* sink, int blocks, int iters, void* stream);

/* Static English text for a status code; never NULL. */
const char* jl_status_string(int status);

/* hipError_t of the most recent JL_EHIP on the calling thread (0 if none). */
int jl_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* BIFOCAL_H */
