/*
 * Seeded synthetic-input generator: the one definition shared by the host
 * (C, gcc) and device (HIP, gfx950) builds of the input generator.
 *
 * It holds no arithmetic of the MoE block. It only turns (seed, tensor id,
 * element index) into a reproducible approximately-N(0, sigma^2) value, so the
 * CPU oracle and the GPU path can be fed identical inputs without copying them
 * between the two.
 *
 * Definition (every step is an integer operation or a single correctly
 * rounded IEEE-754 operation, so host and device agree bit for bit):
 *   1. Stream key   K   = mix64(seed + G * (tensor_id + 1))
 *   2. Element bits u_i = mix64(K + G * (i + 1))
 *      i.e. the (i+1)-th output of SplitMix64 started from state K
 *      (Steele, Lea & Flood, "Fast splittable pseudorandom number
 *      generators", OOPSLA 2014); G = 0x9E3779B97F4A7C15, mix64 is its
 *      output finaliser.
 *   3. Standard normal z by inverse-CDF sampling from a 2^16-cell quantile
 *      table q[0..65536] (q[j] = Phi^-1(j / 65536), ends clamped at
 *      Phi^-1(2^-20)): j = u >> 48, f = ((u >> 16) mod 2^32) * 2^-32,
 *      z = q[j] + (q[j+1] - q[j]) * f  (three separate double operations).
 *      The table is built once on the host and handed to both sides.
 *   4. fp32 value  v = (float)(z * sigma)      (double multiply, then RNE)
 *   5. bf16 value  = round-to-nearest-even of v's upper 16 bits.
 * FMA contraction must be off wherever this header is compiled.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#define SYNTH_FN __host__ __device__ static inline
#else
#define SYNTH_FN static inline
#endif

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL
#define SYNTH_TABLE_CELLS 65536u
#define SYNTH_TABLE_LEN (SYNTH_TABLE_CELLS + 1u)

SYNTH_FN uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

SYNTH_FN uint64_t synth_stream_key(uint64_t seed, uint32_t tensor_id) {
  return synth_mix64(seed + SYNTH_GAMMA * ((uint64_t)tensor_id + 1ULL));
}

SYNTH_FN uint64_t synth_bits(uint64_t key, uint64_t i) {
  return synth_mix64(key + SYNTH_GAMMA * (i + 1ULL));
}

SYNTH_FN double synth_normal(const double* q, uint64_t u) {
#if defined(__clang__)
#pragma clang fp contract(off)
#endif
  uint32_t j = (uint32_t)(u >> 48);
  double f = (double)(uint32_t)(u >> 16) * 0x1p-32; /* exact: 32-bit integer times 2^-32 */
  double lo = q[j];
  double hi = q[j + 1];
  double step = hi - lo;
  double t = step * f;
  return lo + t;
}

SYNTH_FN float synth_scale_f32(double z, double sigma) {
#if defined(__clang__)
#pragma clang fp contract(off)
#endif
  double v = z * sigma;
  return (float)v;
}

SYNTH_FN uint16_t synth_f32_to_bf16(float v) {
  uint32_t b;
  memcpy(&b, &v, 4);
  uint32_t lsb = (b >> 16) & 1u;
  b += 0x7FFFu + lsb; /* values are finite and far from overflow */
  return (uint16_t)(b >> 16);
}

#endif /* SYNTH_CORE_H */
