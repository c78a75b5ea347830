// Host-side check of the FP8 quantiser's scalar helpers (csrc/fp8_codec.h), built with the host
// sanitizers (AddressSanitizer, UndefinedBehaviorSanitizer) by the CPU test suite. Exit status 0
// and a last line "fp8_codec_check ok" mean every check held.
//
// References the helpers are checked against, written from the definitions:
//   - the column scale exponent: the smallest integer e with amax * 2^-e <= 448, found by a plain
//     search in double over every e the float range can need;
//   - the code: the nearest of the 127 non-negative finite e4m3 values (sign, 4 exponent bits
//     biased by 7, 3 mantissa bits, subnormals below 2^-6), ties to the even code, by exhaustive
//     search in double.
#include <float.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "fp8_codec.h"

using moe::fp8::e4m3_rne;
using moe::fp8::scale_exp;

static int failures = 0;
#define CHECK(cond, ...)                \
  do {                                  \
    if (!(cond)) {                      \
      ++failures;                       \
      if (failures < 20) {              \
        fprintf(stderr, "FAIL: ");      \
        fprintf(stderr, __VA_ARGS__);   \
        fprintf(stderr, "\n");          \
      }                                 \
    }                                   \
  } while (0)

static double e4m3_value(int code) {
  const int e = (code >> 3) & 15, m = code & 7;
  const double v = e == 0 ? m / 8.0 * ldexp(1.0, -6) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  return (code & 0x80) ? -v : v;
}

static int ref_code(double v) {
  const double a = fabs(v);
  int best = 0;
  for (int c = 1; c <= 126; ++c) {
    const double dc = fabs(e4m3_value(c) - a), db = fabs(e4m3_value(best) - a);
    if (dc < db || (dc == db && (c % 2 == 0) && (best % 2 == 1))) best = c;
  }
  return (v < 0 && best != 0) ? (best | 0x80) : best;
}

static int ref_exp(double amax) {
  for (int e = -200; e <= 200; ++e)
    if (amax * ldexp(1.0, -e) <= 448.0) return e;
  return 9999;
}

int main() {
  // scale exponent: zero, subnormals, powers of two, the 1.75 boundary and its neighbours,
  // FLT_MAX, and a sweep of random magnitudes
  int e;
  CHECK(scale_exp(0.f, &e) && e == 0, "scale_exp(0)");
  CHECK(!scale_exp(INFINITY, &e), "scale_exp(inf) must report no scale");
  CHECK(!scale_exp(NAN, &e), "scale_exp(nan) must report no scale");
  const float specials[] = {FLT_TRUE_MIN, FLT_MIN, 448.f, 448.f * 1.0000001f, 1.75f, 1.7500001f, 1.7499999f,
                            1.f, 2.f, 3.5f, 0x1p-126f, 0x1.cp-130f, 0x1.c00002p-130f, FLT_MAX, 1e30f, 1e-30f};
  for (float a : specials) {
    const bool ok = scale_exp(a, &e);
    CHECK(ok && e == ref_exp(a), "scale_exp(%a) = %d, want %d", (double)a, e, ref_exp(a));
  }
  srand(7);
  for (int i = 0; i < 200000; ++i) {
    const float a = ldexpf((float)(rand() % (1 << 24) + 1) / (float)(1 << 24), rand() % 276 - 150);
    if (!(a > 0.f) || isinf(a)) continue;
    const bool ok = scale_exp(a, &e);
    CHECK(ok && e == ref_exp(a), "scale_exp(%a) = %d, want %d", (double)a, e, ref_exp(a));
    // and the scaled maximum then rounds to a finite code
    CHECK(e4m3_rne(ldexpf(a, -e)) != 0x7F, "max of a column scaled by 2^%d gives the NaN code", e);
  }

  // codes: every finite code maps to itself, with either sign
  for (int c = 0; c <= 126; ++c) {
    const float v = (float)e4m3_value(c);
    CHECK(e4m3_rne(v) == c, "code %d -> %d", c, e4m3_rne(v));
    if (c) CHECK(e4m3_rne(-v) == (c | 0x80), "code -%d -> %d", c, e4m3_rne(-v));
  }
  // midpoints between neighbouring codes go to the even one; values just off them to the nearer
  for (int c = 0; c < 126; ++c) {
    const double mid = 0.5 * (e4m3_value(c) + e4m3_value(c + 1));
    const float fm = (float)mid;
    if ((double)fm != mid) continue;
    const int want = (c % 2 == 0) ? c : c + 1;
    CHECK(e4m3_rne(fm) == want, "midpoint %a of codes %d, %d -> %d", mid, c, c + 1, e4m3_rne(fm));
    CHECK(e4m3_rne(nextafterf(fm, 0.f)) == c, "just below midpoint %a", mid);
    CHECK(e4m3_rne(nextafterf(fm, 1e9f)) == c + 1, "just above midpoint %a", mid);
  }
  // random values in range against the exhaustive search
  for (int i = 0; i < 200000; ++i) {
    const float v = ((rand() & 1) ? -1.f : 1.f) * 448.f * (float)rand() / (float)RAND_MAX;
    const float w = ldexpf(v, -(rand() % 20));
    CHECK(e4m3_rne(w) == ref_code(w), "e4m3_rne(%a) = %d, want %d", (double)w, e4m3_rne(w), ref_code(w));
  }
  // non-finite and out-of-range inputs: the NaN code with the input's sign, never a trap
  CHECK(e4m3_rne(NAN) == 0x7F || e4m3_rne(NAN) == 0xFF, "nan");
  CHECK(e4m3_rne(INFINITY) == 0x7F, "+inf");
  CHECK(e4m3_rne(-INFINITY) == 0xFF, "-inf");
  CHECK(e4m3_rne(FLT_MAX) == 0x7F, "FLT_MAX");
  CHECK(e4m3_rne(-FLT_MAX) == 0xFF, "-FLT_MAX");
  CHECK(e4m3_rne(449.f) == 0x7F, "449");
  CHECK(e4m3_rne(-0.f) == 0, "-0");
  CHECK(e4m3_rne(FLT_TRUE_MIN) == 0, "smallest subnormal float");

  if (failures) {
    fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  printf("fp8_codec_check ok\n");
  return 0;
}
