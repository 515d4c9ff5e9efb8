// Host-side driver for the sanitizer build of libbifocal's C-ABI layer: every
// call below returns from argument validation, a size query or a host-only
// function, before any HIP call, so the program runs without a GPU. Built
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code, it
// checks that those paths read no memory they do not own and do no signed
// overflow, shift or conversion with undefined behaviour, also at extreme
// sizes. Prints one line per failed expectation; exit status 1 if any.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "bifocal.h"

static int failures = 0;

#define EXPECT_EQ(expr, want)                                                          \
  do {                                                                                 \
    const long long got_ = (long long)(expr);                                          \
    if (got_ != (long long)(want)) {                                                   \
      std::printf("FAIL %s:%d: %s = %lld, expected %lld\n", __FILE__, __LINE__, #expr, \
                  got_, (long long)(want));                                            \
      ++failures;                                                                      \
    }                                                                                  \
  } while (0)

#define EXPECT_TRUE(expr)                                                   \
  do {                                                                      \
    if (!(expr)) {                                                          \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #expr);           \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

static const int64_t I64MAX = INT64_MAX, I64MIN = INT64_MIN;
static const int I32MAX = INT32_MAX, I32MIN = INT32_MIN;

// a non-null address the validation never dereferences
static void* const P = (void*)(uintptr_t)4096;
static const int32_t* const PI = (const int32_t*)(uintptr_t)4096;

static void group_size_and_tiles() {
  EXPECT_EQ(jl_group_size(1, 1), 1);
  EXPECT_EQ(jl_group_size(131072, 32768), 4);
  EXPECT_EQ(jl_group_size(131073, 32768), 5);
  EXPECT_EQ(jl_group_size(I64MAX, 1), I64MAX);
  EXPECT_EQ(jl_group_size(I64MAX, I64MAX), 1);
  EXPECT_EQ(jl_group_size(I64MAX - 1, I64MAX), 1);
  EXPECT_EQ(jl_group_size(0, 5), JL_EINVAL);
  EXPECT_EQ(jl_group_size(5, 0), JL_EINVAL);
  EXPECT_EQ(jl_group_size(I64MIN, 5), JL_EINVAL);
  EXPECT_EQ(jl_group_size(5, I64MIN), JL_EINVAL);
  // tile classes at the ends of the int64 range
  EXPECT_TRUE(jl_tile_class(0, 63, 0, 63, 0) >= 0);
  EXPECT_TRUE(jl_tile_class(I64MAX - 64, I64MAX, 0, 63, I64MAX) >= 0);
  EXPECT_TRUE(jl_tile_class(I64MAX - 64, I64MAX, 0, 63, 0) >= 0);
  EXPECT_EQ(jl_tile_class(10, 5, 0, 1, 0), JL_EINVAL);
  EXPECT_EQ(jl_tile_class(0, 1, 10, 5, 0), JL_EINVAL);
  EXPECT_EQ(jl_tile_class(-1, 1, 0, 1, 0), JL_EINVAL);
  EXPECT_EQ(jl_tile_class(0, 1, 0, 1, -1), JL_EINVAL);
  int bm = 0, bn = 0;
  EXPECT_EQ(jl_prefill_tile_shape(JL_BF16, 128, &bm, &bn), 0);
  EXPECT_TRUE(bm > 0 && bn > 0);
  EXPECT_EQ(jl_prefill_tile_shape(JL_BF16, 128, nullptr, &bn), JL_EINVAL);
  EXPECT_EQ(jl_prefill_tile_shape(JL_BF16, 96, &bm, &bn), JL_EUNSUPPORTED);
  EXPECT_EQ(jl_prefill_tile_shape((jl_dtype)7, 128, &bm, &bn), JL_EUNSUPPORTED);
}

static void status_strings() {
  for (int s = -40; s <= 40; ++s) {
    const char* t = jl_status_string(s);
    EXPECT_TRUE(t != nullptr && std::strlen(t) > 0);
  }
  EXPECT_TRUE(jl_status_string(I32MIN) != nullptr);
  EXPECT_TRUE(jl_status_string(I32MAX) != nullptr);
}

// Size queries: 0 for arguments they reject, no overflow at any size.
static void workspace_sizes() {
  const int64_t Ts[] = {0, 1, 63, 64, 65, 131072, I32MAX / 2, I32MAX, (int64_t)1 << 40, I64MAX,
                        -1, I64MIN};
  const int Bs[] = {1, 2, 4096, I32MAX, 0, -1};
  const int heads[][2] = {{32, 8}, {8, 8}, {2, 1}, {I32MAX, 1}, {0, 1}, {4, 0}, {-4, 2}};
  const int ds[] = {128, 64, 96, 0, -128, I32MAX};
  for (int64_t T : Ts)
    for (int B : Bs)
      for (auto& h : heads)
        for (int d : ds)
          for (int dt = 0; dt < 2; ++dt)
            for (int mode = 0; mode < 3; ++mode) {
              const size_t a = jl_prefill_workspace_size(T, B, h[0], h[1], d, (jl_dtype)dt,
                                                         (jl_mode)mode);
              const size_t c = jl_prefill_workspace_size(T, B, h[0], h[1], d, (jl_dtype)dt,
                                                         (jl_mode)(mode | JL_REMAP_CONTINUOUS));
              EXPECT_EQ(a, c);
              (void)jl_prefill_ie_ratio_offset(T, B, h[0], h[1], d, (jl_dtype)dt);
              (void)jl_prefill_cached_workspace_size(T, T, h[0], h[1], d, (jl_mode)mode);
              (void)jl_decode_workspace_size(T, h[0], d);
              (void)jl_decode_batch_workspace_size(B, T, h[0], d);
            }
  EXPECT_EQ(jl_prefill_workspace_size(-1, 1, 8, 2, 128, JL_BF16, JL_MODE_FUSED), 0);
  EXPECT_EQ(jl_decode_workspace_size(0, 8, 128), 0);
  EXPECT_EQ(jl_decode_batch_workspace_size(0, 10, 8, 128), 0);
  EXPECT_TRUE(jl_prefill_workspace_size(131072, 1, 32, 8, 128, JL_BF16, JL_MODE_FUSED) > 0);
  EXPECT_TRUE(jl_decode_workspace_size(131072, 32, 128) > 0);
}

static int prefill(const int32_t* cu, int B, int64_t T, int Hq, int Hkv, int d, int64_t w0,
                   int64_t w_pre, double theta, float scale, int dt, int mode, void* ws,
                   size_t ws_bytes, void* x = P) {
  return jl_bifocal_prefill(x, P, P, P, nullptr, nullptr, cu, B, T, Hq, Hkv, d, w0, w_pre, theta,
                            scale, (jl_dtype)dt, (jl_mode)mode, ws, ws_bytes, nullptr);
}

static void prefill_errors() {
  const size_t big = (size_t)1 << 50;
  EXPECT_EQ(prefill(nullptr, 1, 256, 3, 2, 128, 16, 64, 1e4, 0.f, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 1, 256, 4, 0, 128, 16, 64, 1e4, 0.f, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 1, -1, 4, 2, 128, 16, 64, 1e4, 0.f, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 1, I64MIN, 4, 2, 128, 16, 64, 1e4, 0.f, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 1, I64MAX, 4, 2, 128, 16, 64, 1e4, 0.f, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 1, 256, 4, 2, 128, -1, 64, 1e4, 0.f, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 1, 256, 4, 2, 128, I64MIN, 64, 1e4, 0.f, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 1, 256, 4, 2, 128, 16, 0, 1e4, 0.f, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 1, 256, 4, 2, 128, 16, 64, 1.0, 0.f, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 1, 256, 4, 2, 128, 16, 64, 0.0 / 0.0, 0.f, 0, 0, P, big),
            JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 1, 256, 4, 2, 128, 16, 64, 1e4, 0.f / 0.f, 0, 0, P, big),
            JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 2, 256, 4, 2, 128, 16, 64, 1e4, 0.f, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 1, 256, 4, 2, 96, 16, 64, 1e4, 0.f, 0, 0, P, big), JL_EUNSUPPORTED);
  EXPECT_EQ(prefill(nullptr, 1, 256, 4, 2, I32MAX, 16, 64, 1e4, 0.f, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 1, 256, 4, 2, 128, 16, 64, 1e4, 0.f, 0, 7, P, big), JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 1, 256, 4, 2, 128, 16, 64, 1e4, 0.f, 0, 32, P, big), JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 1, 256, 4, 2, 128, 16, 64, 1e4, 0.f, 5, 0, P, big), JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 1, 256, 4, 2, 128, 16, 64, 1e4, 0.f, 0, 0, P, big, nullptr),
            JL_EINVAL);
  EXPECT_EQ(prefill(nullptr, 1, 256, 4, 2, 128, 16, 64, 1e4, 0.f, 0, 0, nullptr, big),
            JL_EWORKSPACE);
  EXPECT_EQ(prefill(nullptr, 1, 256, 4, 2, 128, 16, 64, 1e4, 0.f, 0, 0, P, 10), JL_EWORKSPACE);
  EXPECT_EQ(prefill(nullptr, 1, 256, 4, 2, 128, 16, 64, 1e4, 0.f, 0, 0,
                    (void*)((uintptr_t)P + 8), big),
            JL_EINVAL);
  EXPECT_EQ(prefill(PI, 5000, 256, 4, 2, 128, 16, 64, 1e4, 0.f, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(prefill(PI, I32MAX, 256, 4, 2, 128, 16, 64, 1e4, 0.f, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(prefill(PI, I32MIN, 256, 4, 2, 128, 16, 64, 1e4, 0.f, 0, 0, P, big), JL_EINVAL);
  // T == 0 returns before touching anything
  EXPECT_EQ(jl_bifocal_prefill(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1,
                               0, 4, 2, 128, 16, 64, 1e4, 0.f, JL_BF16, JL_MODE_FUSED, nullptr, 0,
                               nullptr),
            0);
}

static int cached(int64_t q_off, int64_t Tq, int64_t cap, int Hq, int Hkv, int d, int64_t w0,
                  int64_t w_pre, double theta, int dt, int mode, void* ws, size_t ws_bytes) {
  return jl_bifocal_prefill_cached(P, P, P, P, nullptr, q_off, Tq, cap, Hq, Hkv, d, w0, w_pre,
                                   theta, 0.f, (jl_dtype)dt, (jl_mode)mode, ws, ws_bytes,
                                   nullptr);
}

static void cached_errors() {
  const size_t big = (size_t)1 << 50;
  EXPECT_EQ(cached(-1, 50, 1000, 8, 2, 128, 16, 64, 1e4, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(cached(100, -1, 1000, 8, 2, 128, 16, 64, 1e4, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(cached(960, 50, 1000, 8, 2, 128, 16, 64, 1e4, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(cached(I64MAX, 1, I64MAX, 8, 2, 128, 16, 64, 1e4, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(cached(1, I64MAX, I64MAX, 8, 2, 128, 16, 64, 1e4, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(cached(I64MAX, I64MAX, I64MAX, 8, 2, 128, 16, 64, 1e4, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(cached(100, 50, 0, 8, 2, 128, 16, 64, 1e4, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(cached(100, 50, 1000, 6, 4, 128, 16, 64, 1e4, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(cached(100, 50, 1000, 8, 2, 128, I64MIN, 64, 1e4, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(cached(100, 50, 1000, 8, 2, 128, 16, 64, 1e4, 0, 1, P, big), JL_EUNSUPPORTED);
  EXPECT_EQ(cached(100, 50, 1000, 8, 2, 64, 16, 64, 1e4, 0, 0, P, big), JL_EUNSUPPORTED);
  EXPECT_EQ(cached(100, 50, 1000, 8, 2, 128, 16, 64, 1e4, 4, 0, P, big), JL_EINVAL);
  EXPECT_EQ(cached(100, 50, 1000, 8, 2, 128, 16, 64, 1e4, 0, 0, nullptr, big), JL_EWORKSPACE);
  EXPECT_EQ(cached(100, 50, 1000, 8, 2, 128, 16, 64, 1e4, 0, 0, P, 64), JL_EWORKSPACE);
  EXPECT_EQ(cached(0, 0, 1000, 8, 2, 128, 16, 64, 1e4, 0, 0, nullptr, 0), 0);
}

static int decode(int64_t pos, int64_t cap, int Hq, int Hkv, int d, int64_t w0, int64_t w_pre,
                  double theta, int dt, int mode, int splits, void* ws, size_t ws_bytes) {
  return jl_bifocal_decode(P, P, P, P, nullptr, pos, cap, Hq, Hkv, d, w0, w_pre, theta, 0.f,
                           (jl_dtype)dt, (jl_mode)mode, splits, ws, ws_bytes, nullptr);
}

static void decode_errors() {
  const size_t big = (size_t)1 << 50;
  EXPECT_EQ(decode(-1, 1000, 8, 2, 128, 16, 64, 1e4, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(decode(1000, 1000, 8, 2, 128, 16, 64, 1e4, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(decode(I64MAX, I64MAX, 8, 2, 128, 16, 64, 1e4, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(decode(5, I64MAX, 8, 2, 128, 16, 64, 1e4, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(decode(100, 0, 8, 2, 128, 16, 64, 1e4, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(decode(100, 1000, 6, 4, 128, 16, 64, 1e4, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(decode(100, 1000, I32MIN, 2, 128, 16, 64, 1e4, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(decode(100, 1000, 8, 2, 128, -2, 64, 1e4, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(decode(100, 1000, 8, 2, 128, 16, 0, 1e4, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(decode(100, 1000, 8, 2, 128, 16, 64, 1e4, 0, 0, -1, P, big), JL_EINVAL);
  EXPECT_EQ(decode(100, 1000, 8, 2, 128, 16, 64, 1e4, 0, 0, I32MAX, P, big), JL_EINVAL);
  EXPECT_EQ(decode(100, 1000, 8, 2, 128, 16, 64, 1e4, 0, 1, 0, P, big), JL_EUNSUPPORTED);
  EXPECT_EQ(decode(100, 1000, 8, 2, 128, 16, 64, 1e4, 0, 9, 0, P, big), JL_EINVAL);
  EXPECT_EQ(decode(100, 1000, 8, 2, 96, 16, 64, 1e4, 0, 0, 0, P, big), JL_EUNSUPPORTED);
  EXPECT_EQ(decode(100, 1000, 12, 4, 128, 16, 64, 1e4, 0, 0, 0, P, big), JL_EUNSUPPORTED);
  EXPECT_EQ(decode(100, 1000, 8, 2, 128, 16, 64, 0.5, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(decode(100, 1000, 8, 2, 128, 16, 64, 1e4, 0, 0, 0, nullptr, big), JL_EWORKSPACE);
  EXPECT_EQ(decode(100, 1000, 8, 2, 128, 16, 64, 1e4, 0, 0, 0, P, 100), JL_EWORKSPACE);
  EXPECT_EQ(decode(100, 1000, 8, 2, 128, I64MAX, I64MAX, 1e300, 0, 0, 0, P, 100), JL_EWORKSPACE);
}

static int batch(int B, int64_t max_keys, int64_t rows, int Hq, int Hkv, int d, int64_t w0,
                 int64_t w_pre, double theta, int dt, int mode, int splits, void* ws,
                 size_t ws_bytes) {
  return jl_bifocal_decode_batch(P, P, P, P, nullptr, PI, PI, B, max_keys, rows, Hq, Hkv, d, w0,
                                 w_pre, theta, 0.f, (jl_dtype)dt, (jl_mode)mode, splits, ws,
                                 ws_bytes, nullptr);
}

static void batch_errors() {
  const size_t big = (size_t)1 << 50;
  EXPECT_EQ(batch(-1, 1000, 5000, 8, 2, 128, 16, 64, 1e4, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(batch(70000, 1000, 5000, 8, 2, 128, 16, 64, 1e4, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(batch(I32MAX, 1000, 5000, 8, 2, 128, 16, 64, 1e4, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(batch(4, 0, 5000, 8, 2, 128, 16, 64, 1e4, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(batch(4, I64MAX, I64MAX, 8, 2, 128, 16, 64, 1e4, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(batch(4, 1000, 0, 8, 2, 128, 16, 64, 1e4, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(batch(4, 1000, 5000, 6, 4, 128, 16, 64, 1e4, 0, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(batch(4, 1000, 5000, 8, 2, 128, 16, 64, 1e4, 0, 0, 5000, P, big), JL_EINVAL);
  EXPECT_EQ(batch(4, 1000, 5000, 8, 2, 128, 16, 64, 1e4, 0, 1, 0, P, big), JL_EUNSUPPORTED);
  EXPECT_EQ(batch(4, 1000, 5000, 8, 2, 96, 16, 64, 1e4, 0, 0, 0, P, big), JL_EUNSUPPORTED);
  EXPECT_EQ(batch(4, 1000, 5000, 8, 2, 128, 16, 64, 1e4, 4, 0, 0, P, big), JL_EINVAL);
  EXPECT_EQ(batch(4, 1000, 5000, 8, 2, 128, 16, 64, 1e4, 0, 0, 0, nullptr, big), JL_EWORKSPACE);
  EXPECT_EQ(batch(4, 1000, 5000, 8, 2, 128, 16, 64, 1e4, 0, 0, 0, P, 100), JL_EWORKSPACE);
  EXPECT_EQ(jl_bifocal_decode_batch(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                    0, 1000, 5000, 8, 2, 128, 16, 64, 1e4, 0.f, JL_BF16,
                                    JL_MODE_FUSED, 0, nullptr, 0, nullptr),
            0);
}

static void rope_and_misc_errors() {
  EXPECT_EQ(jl_rope_apply(P, -1, 2, 128, nullptr, 1, 0, 1e4, JL_BF16, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_rope_apply(P, I64MIN, 2, 128, nullptr, 1, 0, 1e4, JL_BF16, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_rope_apply(P, I64MAX, 2, 128, nullptr, 1, 0, 1e4, JL_BF16, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_rope_apply(P, 10, 0, 128, nullptr, 1, 0, 1e4, JL_BF16, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_rope_apply(P, 10, I32MAX, I32MAX, nullptr, 1, 0, 1e4, JL_BF16, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_rope_apply(P, 10, 2, 7, nullptr, 1, 0, 1e4, JL_BF16, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_rope_apply(P, 10, 2, 40, nullptr, 1, 0, 1e4, JL_BF16, nullptr), JL_EUNSUPPORTED);
  EXPECT_EQ(jl_rope_apply(P, 10, 2, 128, nullptr, 1, -1, 1e4, JL_BF16, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_rope_apply(P, 10, 2, 128, nullptr, 1, I64MIN, 1e4, JL_BF16, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_rope_apply(P, 10, 2, 128, nullptr, 1, 0, 1.0, JL_BF16, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_rope_apply(nullptr, 10, 2, 128, nullptr, 1, 0, 1e4, JL_BF16, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_rope_apply(P, 10, 2, 128, PI, 0, 0, 1e4, JL_BF16, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_rope_apply(nullptr, 0, 2, 128, nullptr, 1, 0, 1e4, JL_BF16, nullptr), 0);
  EXPECT_EQ(jl_debug_tile_classes(0, 0, (int8_t*)P, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_debug_tile_classes(10, -1, (int8_t*)P, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_debug_tile_classes(I64MAX, 0, (int8_t*)P, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_calib_stream_read(nullptr, 1024, (uint32_t*)P, 16, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_calib_stream_read(P, 1000, (uint32_t*)P, 16, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_calib_stream_read(P, 1024, (uint32_t*)P, 0, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_calib_stream_read_ex(P, 1024, (uint32_t*)P, 16, 9, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_calib_stream_read_ex(P, 1024, (uint32_t*)P, 16, -1, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_calib_mfma_bf16(nullptr, 4, 10, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_calib_mfma_bf16((float*)P, 0, 10, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_prefill_flags(nullptr, (uint32_t*)P, nullptr), JL_EINVAL);
  EXPECT_EQ(jl_prefill_flags(P, nullptr, nullptr), JL_EINVAL);
}

int main() {
  group_size_and_tiles();
  status_strings();
  workspace_sizes();
  prefill_errors();
  cached_errors();
  decode_errors();
  batch_errors();
  rope_and_misc_errors();
  std::printf("abi_validation: %d failure(s)\n", failures);
  return failures ? 1 : 0;
}
