// Host-side checks of the C ABI in include/fa.h, built with AddressSanitizer
// and UndefinedBehaviorSanitizer on the host pass (tests/test_cabi_sanitized.py
// builds and runs it; no GPU is needed).  Every call below is rejected by the
// argument validation before anything reaches the GPU: null pointers, sizes
// at the int limits (the size checks must not overflow 64 bits), bad
// windows, strides and split counts, misaligned addresses, and host sign
// arrays exactly d bytes long (the validation must read no further).  The
// pointers are fake addresses that are never dereferenced.
#include <limits.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "../include/fa.h"

static int failures = 0;

#define EXPECT(expr, want)                                                   \
  do {                                                                       \
    const int got_ = (expr);                                                 \
    if (got_ != (want)) {                                                    \
      fprintf(stderr, "FAIL line %d: %s = %d, want %d\n", __LINE__, #expr,   \
              got_, (int)(want));                                            \
      ++failures;                                                            \
    }                                                                        \
  } while (0)

int main() {
  void* const A = reinterpret_cast<void*>(0x10000);     // 16-byte aligned
  void* const M = reinterpret_cast<void*>(0x10008);     // 8-byte aligned
  void* const M4 = reinterpret_cast<void*>(0x10002);    // 2-byte aligned
  float* const Af = static_cast<float*>(A);
  float* const Mf = static_cast<float*>(M);
  const int* const Ai = static_cast<const int*>(A);
  const unsigned* const Au = static_cast<const unsigned*>(A);
  const float s = 0.1f;
  const int BIG = INT_MAX;

  // ---- fa_fwd ----
  EXPECT(fa_fwd(nullptr, A, A, A, Af, 1, 2, 2, 8, 128, 0, s, 0, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd(A, nullptr, A, A, Af, 1, 2, 2, 8, 128, 0, s, 0, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd(A, A, nullptr, A, Af, 1, 2, 2, 8, 128, 0, s, 0, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd(A, A, A, nullptr, Af, 1, 2, 2, 8, 128, 0, s, 0, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd(A, A, A, A, nullptr, 1, 2, 2, 8, 128, 0, s, 0, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd(A, A, A, A, Af, 0, 2, 2, 8, 128, 0, s, 0, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd(A, A, A, A, Af, 1, -2, 2, 8, 128, 0, s, 0, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd(A, A, A, A, Af, 1, 6, 4, 8, 128, 0, s, 0, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd(A, A, A, A, Af, 1, 2, 2, 8, 128, 0, NAN, 0, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd(A, A, A, A, Af, 1, 2, 2, 8, 128, 0, INFINITY, 0, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd(A, A, A, A, Af, BIG, BIG, 1, BIG, 128, 0, s, 0, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd(A, A, A, A, Af, BIG, 1, 1, BIG, 128, 0, s, 0, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd(A, A, A, A, Af, 1, 2, 2, 8, 96, 0, s, 0, nullptr),
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd(A, A, A, A, Af, 1, 2, 2, 8, 128, 0, s, 7, nullptr),
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd(A, A, A, A, Af, 1, 2, 2, 8, 64, 0, s, 1, nullptr),
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd(M, A, A, A, Af, 1, 2, 2, 8, 128, 0, s, 0, nullptr),
         FA_ERR_MISALIGNED);
  EXPECT(fa_fwd(A, A, A, A, Mf, 1, 2, 2, 8, 128, 0, s, 0, nullptr),
         FA_ERR_MISALIGNED);
  EXPECT(fa_fwd(M, A, A, A, Af, 1, 2, 2, 0, 96, 0, s, 0, nullptr),
         FA_ERR_INVALID_ARGUMENT);

  // ---- fa_fwd_fp8 ----
  EXPECT(fa_fwd_fp8(A, A, A, A, Af, BIG, BIG, BIG, BIG, 128, 1, s, nullptr,
                    nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_fp8(A, A, A, A, Af, 1, 2, 2, 8, 64, 0, s, nullptr, nullptr),
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd_fp8(A, A, A, A, Af, 1, 2, 2, 8, 128, 0, s,
                    static_cast<const float*>(M4), nullptr),
         FA_ERR_MISALIGNED);

  // ---- fa_fwd_fp8_exp2_fma, fa_exp2_fma ----
  EXPECT(fa_fwd_fp8_exp2_fma(A, A, A, A, Af, BIG, BIG, BIG, BIG, 128, 1, s,
                             nullptr, 8, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_fp8_exp2_fma(A, A, A, A, Af, 1, 2, 2, 8, 128, 0, s, nullptr,
                             BIG, nullptr),
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd_fp8_exp2_fma(A, A, A, A, Af, 1, 2, 2, 8, 128, 0, s,
                             static_cast<const float*>(M4), 4, nullptr),
         FA_ERR_MISALIGNED);
  EXPECT(fa_exp2_fma(Af, Af, -1, nullptr), FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_exp2_fma(static_cast<const float*>(M4), Af, LLONG_MAX, nullptr),
         FA_ERR_MISALIGNED);

  // ---- fa_bwd ----
  EXPECT(fa_bwd(A, A, A, A, Af, nullptr, A, A, A, Af, 1, 2, 2, 8, 128, 0, s,
                nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_bwd(A, A, A, A, Af, A, A, A, A, nullptr, 1, 2, 2, 8, 128, 0, s,
                nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_bwd(A, A, A, A, Af, A, A, A, A, Af, BIG, BIG, 1, BIG, 128, 0, s,
                nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_bwd(A, A, A, A, Af, A, A, A, A, Af, 1, 2, 2, 8, 64, 0, s,
                nullptr),
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_bwd(A, A, A, A, Af, A, M, A, A, Af, 1, 2, 2, 8, 128, 0, s,
                nullptr),
         FA_ERR_MISALIGNED);

  // ---- fa_fwd_splitkv / fa_splitkv_num_splits ----
  EXPECT(fa_fwd_splitkv(A, A, A, A, Af, 1, 8, 2, 1, 4096, 128, 1, s, 0, Af,
                        nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_splitkv(A, A, A, A, Af, 1, 8, 2, 1, 4096, 128, 1, s, 257, Af,
                        nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_splitkv(A, A, A, A, Af, BIG, BIG, 1, BIG, BIG, 128, 1, s, 4,
                        Af, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_splitkv(A, A, A, A, Af, 1, 8, 2, 1, 4096, 128, 1, s, 4,
                        nullptr, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_splitkv(A, A, A, A, Af, 1, 8, 2, 1, 4096, 64, 1, s, 4, Af,
                        nullptr),
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd_splitkv(A, A, A, A, Af, 1, 8, 2, 1, 4096, 128, 1, s, 4, Mf,
                        nullptr),
         FA_ERR_MISALIGNED);
  {
    const int shapes[][5] = {{8, 32, 8, 1, 65536},  {1, 1, 1, 1, 1},
                             {1, 32, 8, 1, 131072}, {16, 32, 8, 4, 16384},
                             {BIG, BIG, 1, BIG, BIG}, {1, 1, 1, BIG, BIG}};
    for (const auto& sh : shapes) {
      const int n = fa_splitkv_num_splits(sh[0], sh[1], sh[2], sh[3], sh[4]);
      if (n < 1 || n > 256) {
        fprintf(stderr, "FAIL: fa_splitkv_num_splits = %d\n", n);
        ++failures;
      }
    }
    EXPECT(fa_splitkv_num_splits(0, 8, 2, 1, 4096), 0);
    EXPECT(fa_splitkv_num_splits(1, 6, 4, 1, 4096), 0);
  }

  // ---- fa_fwd_splitkv_noalloc ----
  EXPECT(fa_fwd_splitkv_noalloc(nullptr, A, A, A, Af, 1, 8, 2, 1, 4096, 128,
                                1, s, 8, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_splitkv_noalloc(A, A, A, A, Af, BIG, BIG, 1, BIG, 8, 128, 1,
                                s, 8, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_splitkv_noalloc(A, A, A, A, Af, 2, 16, 4, 512, 4096, 128, 1,
                                s, 256, nullptr),
         FA_ERR_WORKSPACE);
  EXPECT(fa_fwd_splitkv_noalloc(A, A, A, A, Af, 1 << 20, 1 << 10, 1, 1, 8,
                                128, 1, s, 256, nullptr),
         FA_ERR_WORKSPACE);

  // ---- fa_fwd_varlen ----
  EXPECT(fa_fwd_varlen(A, A, A, A, Af, Ai, nullptr, 2, 4, 2, 100, 100, 64,
                       128, 1, -1, -1, s, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_varlen(A, A, A, A, Af, Ai, Ai, 2, 4, 2, 100, 100, 64, 128, 0,
                       -2, -1, s, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_varlen(A, A, A, A, Af, Ai, Ai, 2, 4, 2, 100, 100, 64, 128, 0,
                       -1, INT_MIN, s, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_varlen(A, A, A, A, Af, Ai, Ai, 2, 4, 2, (1 << 29) + 1, 100,
                       64, 128, 0, -1, -1, s, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_varlen(A, A, A, A, Af, Ai, Ai, 2, BIG, 1, BIG, BIG, BIG, 128,
                       0, BIG, BIG, s, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_varlen(A, A, A, A, Af, Ai, Ai, 2, 4, 2, 100, 100, 64, 64, 0,
                       BIG, BIG, s, nullptr),
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd_varlen(A, A, A, A, static_cast<float*>(M4), Ai, Ai, 2, 4, 2,
                       100, 100, 64, 128, 0, BIG, BIG, s, nullptr),
         FA_ERR_MISALIGNED);
  EXPECT(fa_fwd_varlen(A, A, A, A, Af, static_cast<const int*>(M4), Ai, 2, 4,
                       2, 100, 100, 64, 128, 0, BIG, 0, s, nullptr),
         FA_ERR_MISALIGNED);

  // ---- fa_fwd_masked ----
  EXPECT(fa_fwd_masked(A, A, A, A, Af, nullptr, 0, 0, 1, 2, 2, 8, 8, 128, s,
                       nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_masked(A, A, A, A, Af, Au, -1, 0, 1, 2, 2, 8, 8, 128, s,
                       nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_masked(A, A, A, A, Af, Au, 0, 0, BIG, BIG, 1, BIG, 8, 128, s,
                       nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fwd_masked(A, A, A, A, Af, Au, 0, 0, 1, 2, 2, 8, 262145, 128, s,
                       nullptr),
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd_masked(A, A, A, A, Af, static_cast<const unsigned*>(M4), 0, 0,
                       1, 2, 2, 8, 8, 128, s, nullptr),
         FA_ERR_MISALIGNED);

  // ---- fa_fp8_quantize: host sign arrays of exactly d entries ----
  for (int d : {1, 64, 127, 128, 200}) {
    signed char* good = static_cast<signed char*>(malloc(d));
    signed char* bad = static_cast<signed char*>(malloc(d));
    for (int i = 0; i < d; ++i) {
      good[i] = (i % 3) ? 1 : -1;
      bad[i] = 1;
    }
    bad[d - 1] = (d <= 128) ? 0 : 1;     // an invalid entry the check reads
    // Valid signs pass the checks; the misaligned input then stops the
    // call (d == 128) or the unsupported d does, before any launch.
    const float* x = static_cast<const float*>(M);
    EXPECT(fa_fp8_quantize(x, A, Af, 4, d, good, nullptr),
           d == 128 ? FA_ERR_MISALIGNED : FA_ERR_UNSUPPORTED);
    if (d <= 128)
      EXPECT(fa_fp8_quantize(x, A, Af, 4, d, bad, nullptr),
             FA_ERR_INVALID_ARGUMENT);
    free(good);
    free(bad);
  }
  EXPECT(fa_fp8_quantize(nullptr, A, Af, 4, 128, nullptr, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fp8_quantize(static_cast<const float*>(A), A, Af, 0, 128, nullptr,
                         nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fp8_quantize(static_cast<const float*>(A), A, Af, (1LL << 40) + 1,
                         128, nullptr, nullptr),
         FA_ERR_INVALID_ARGUMENT);
  EXPECT(fa_fp8_quantize(static_cast<const float*>(M), A, Af, 4, 128, nullptr,
                         nullptr),
         FA_ERR_MISALIGNED);

  // ---- sizes that pass the checks but not a launcher's 32-bit offsets ----
  // One (batch, head) of 2^31 - 1 rows: each launcher refuses before any
  // launch and the call reports FA_ERR_HIP with the HIP error behind it.
  EXPECT(fa_last_hip_error(), 0);
  EXPECT(fa_fwd(A, A, A, A, Af, 1, 1, 1, BIG, 128, 0, s, 0, nullptr),
         FA_ERR_HIP);
  EXPECT(fa_fwd(A, A, A, A, Af, 1, 1, 1, BIG, 64, 1, s, 0, nullptr),
         FA_ERR_HIP);
  EXPECT(fa_fwd_fp8(A, A, A, A, Af, 1, 1, 1, BIG, 128, 1, s, nullptr,
                    nullptr),
         FA_ERR_HIP);
  EXPECT(fa_bwd(A, A, A, A, Af, A, A, A, A, Af, 1, 1, 1, BIG, 128, 1, s,
                nullptr),
         FA_ERR_HIP);
  if (fa_last_hip_error() == 0) {
    fprintf(stderr, "FAIL: fa_last_hip_error() is 0 after FA_ERR_HIP\n");
    ++failures;
  }

  // ---- status plumbing ----
  for (int st = -3; st < 10; ++st) {
    if (fa_status_string(st) == nullptr) {
      fprintf(stderr, "FAIL: fa_status_string(%d) is NULL\n", st);
      ++failures;
    }
  }
  EXPECT(fa_version(), 100);

  printf("%d failures\n", failures);
  return failures ? 1 : 0;
}
