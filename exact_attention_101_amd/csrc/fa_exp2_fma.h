// 2^x on the FMA pipe: the software exponential that the FlashAttention-4
// article («Оптимизируйте производительность с FlashAttention-4», paragraph
// 3) uses for part of the softmax's exponentials on Blackwell, where the
// exponential unit is slower than the FMA units.  Here it is an option of
// the fp8 forward (a chosen share of each tile's exponentials), measured
// against v_exp_f32.
//
// Method: range reduction x = n + f with n = rint(x) and f in [-1/2, 1/2]
// (exact for base 2; Cody and Waite split the reduction constant only for
// other bases), 2^f from a degree-3 polynomial whose coefficients minimise
// the maximum relative error on [-1/2, 1/2] (Remez exchange, fitted by
// exp2_fit.py beside this file: float32 Horner evaluation within 7.5e-5
// relative), and the scale 2^n added to the exponent field.
//
// Instructions: v_max_f32, v_add_f32, two v_sub_f32, three v_fma_f32 and
// v_lshl_add_u32 -- eight full-rate vector instructions against one
// v_exp_f32.
//
// Domain: x <= 127 (the result is then a normal float within 7.5e-5 of
// 2^x, relative).  x < -125, -inf included, returns 2^-125 * p(0), about
// 2.35e-38, instead of rounding to zero: a consumer that rounds it to e4m3
// (smallest subnormal 2^-9) or adds it to a sum of order one loses it.
#ifndef FA_EXP2_FMA_H_
#define FA_EXP2_FMA_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Remez coefficients of 2^f on [-1/2, 1/2], c0 first (exp2_fit.py 3).
constexpr float EXP2_C0 = 0x1.fff692p-1f;
constexpr float EXP2_C1 = 0x1.62f31ap-1f;
constexpr float EXP2_C2 = 0x1.f0de1ap-3f;
constexpr float EXP2_C3 = 0x1.c3f76p-5f;

__device__ __forceinline__ float exp2_fma(float x) {
  // 1.5 * 2^23: adding it rounds x to an integer n held in the low
  // mantissa bits of t (|x| < 2^22), so that bits(t) << 23 is n << 23.
  constexpr float ROUND = 12582912.0f;
  x = fmaxf(x, -125.0f);
  const float t = x + ROUND;
  const float n = t - ROUND;
  const float f = x - n;
  float p = fmaf(EXP2_C3, f, EXP2_C2);
  p = fmaf(p, f, EXP2_C1);
  p = fmaf(p, f, EXP2_C0);
  return __uint_as_float(__float_as_uint(p) + (__float_as_uint(t) << 23));
}

}  // namespace fa

#endif  // FA_EXP2_FMA_H_
