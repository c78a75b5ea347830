// Scalar helpers of the FP8 weight quantiser, compiled for the device (the quantiser kernel) and
// for the host (a sanitized CPU check of exactly these functions).
//
// Format: OCP e4m3 -- sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
// infinities, largest finite value 448 (code 0x7E), NaN codes 0x7F and 0xFF. The Fondations page
// of the Qwen3.8-Max report names FP8 among the formats without fixing a scheme; the scheme used
// here is one power-of-two scale per output column and round to nearest, ties to even.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace moe {
namespace fp8 {

constexpr float kE4m3Max = 448.0f;
constexpr uint8_t kE4m3NaN = 0x7F;

// Exponent e of a column's scale 2^e: the smallest integer e with amax * 2^-e <= 448, and 0 for an
// all-zero column (amax == 0). Write amax = f * 2^E with f in [1, 2) (E = ilogb(amax), subnormals
// included). For e >= E - 7, amax * 2^-e < 2^8 <= 448; for e = E - 8 the bound reads f * 2^8 <= 448,
// i.e. f <= 1.75; for e <= E - 9 it fails. So e = E - 8 when f <= 1.75 and E - 7 otherwise: a
// closed form, no search. A non-finite amax (the column holds an Inf or a NaN) has no such e: the
// function returns false and the caller gives the column a NaN scale.
__host__ __device__ inline bool scale_exp(float amax, int* e) {
  if (!(amax >= 0.f) || amax == INFINITY) {  // NaN or +Inf (amax is a maximum of magnitudes)
    *e = 0;
    return false;
  }
  if (amax == 0.f) {
    *e = 0;
    return true;
  }
  const int E = ilogbf(amax);
  const float f = ldexpf(amax, -E);  // exact: a power-of-two scaling into [1, 2)
  *e = f <= 1.75f ? E - 8 : E - 7;
  return true;
}

// Nearest e4m3 code of v, ties to the even code. Callers scale into range (|v| <= 448); anything
// else -- NaN, an infinity or a larger magnitude -- gets the NaN code with v's sign.
//   |v| < 2^-6 (subnormal range): v is a multiple of 2^-9 times the mantissa code; rint of
//     |v| * 2^9 rounds to nearest even, and 8 -- the smallest normal's code -- is reached exactly
//     when rounding carries out of the subnormals.
//   otherwise |v| in [2^E, 2^(E+1)): |v| * 2^(3-E) lies in [8, 16); rint gives 8 + m, and m = 8 is a
//     carry into the next binade (m = 0, E + 1).
// Every scaling is by a power of two, so the only rounding is the one rint performs (the default
// round-to-nearest-even mode).
__host__ __device__ inline uint8_t e4m3_rne(float v) {
  const uint8_t sign = signbit(v) ? 0x80u : 0u;
  const float a = fabsf(v);
  if (!(a <= kE4m3Max)) return (uint8_t)(kE4m3NaN | sign);
  int code;
  if (a < 0x1p-6f) {
    code = (int)rintf(a * 512.0f);
  } else {
    const int E = ilogbf(a);
    int m = (int)rintf(ldexpf(a, 3 - E)) - 8;  // 0 .. 8
    int EE = E;
    if (m == 8) {
      m = 0;
      EE += 1;
    }
    code = ((EE + 7) << 3) | m;
  }
  return code == 0 ? (uint8_t)0 : (uint8_t)(code | sign);
}

}  // namespace fp8
}  // namespace moe
