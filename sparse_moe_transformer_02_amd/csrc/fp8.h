// E4M3FN encoding on the device, written from the format's bit layout.
//
// E4M3FN: sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is subnormal with
// step 2^-9; the largest finite magnitude is 448 (exponent 15, mantissa 6); no infinities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Round-to-nearest-even, saturating at +-448, sign copied from the input (so -0 -> 0x80).
// Inputs at or above 448 in magnitude (and non-finite ones) give 0x7E / 0xFE.
__device__ __forceinline__ uint32_t e4m3_encode(float q) {
  const uint32_t b = __float_as_uint(q);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x43e00000u) {                       // |q| >= 448
    code = 0x7eu;
  } else if (a < 0x3c800000u) {                 // |q| < 2^-6: subnormal grid, step 2^-9
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);   // exact scaling, RNE; 8 = 2^-6
  } else {                                      // normal: keep 3 of 23 mantissa bits, ties to even
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);             // (fp32 exponent - 127 + 7) << 3 | mantissa
  }
  return sign | code;
}

}  // namespace moe
