// OCP E4M3 encoding with power-of-two scales, shared by the FP8 cache's writer (the memory
// update) and the FP8 attention's chunk quantization.
#pragma once

#include "common.h"

namespace pbsa {

// OCP E4M3 code of y (|y| <= 448, finite) nearest to it, ties to the even mantissa: the
// subnormal codes are the multiples of 2^-9 below 2^-6 (rounded by v_rndne), the normal
// ones keep 3 mantissa bits of y's fp32 mantissa, rounded to nearest even.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a < 0x3c800000u) {  // |y| < 2^-6
    code = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.f));
  } else {
    int ee = static_cast<int>(a >> 23) - 127 + 7;  // biased E4M3 exponent, >= 1
    uint32_t m = (a >> 20) & 7u;
    const uint32_t rem = a & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ++m;
    if (m == 8u) {
      m = 0;
      ++ee;
    }
    code = (static_cast<uint32_t>(ee) << 3) | m;
  }
  return sign | code;
}

// The smallest power of two 2^e with amax <= 448 * 2^e (1 for amax = 0): with
// amax = f * 2^E, f in [0.5, 1), and 448 = 0.875 * 2^9, e = E - 9 when f <= 0.875, else
// E - 8.
__device__ __forceinline__ int e4m3_scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float f = frexpf(amax, &E);
  return f <= 0.875f ? E - 9 : E - 8;
}

}  // namespace pbsa
