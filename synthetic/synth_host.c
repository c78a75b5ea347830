/*
 * Host side of the seeded synthetic-input generator (see synth_core.h for the
 * definition). Built with gcc -ffp-contract=off -fopenmp into
 * libsynth_host.so; no GPU needed.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#include "synth_core.h"

/* Phi(x) for the standard normal, from libm's erfc. */
static double std_normal_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/* Phi^-1(p) for 0 < p <= 1/2 by bisection on [-40, 0]; 200 halvings reach
 * adjacent doubles, so the result is a deterministic function of libm. */
static double std_normal_quantile_lower(double p) {
  double lo = -40.0, hi = 0.0;
  for (int it = 0; it < 200; ++it) {
    double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (std_normal_cdf(mid) < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

/* q[j] = Phi^-1(j / 65536) for 1 <= j <= 65535, q[0] = Phi^-1(2^-20),
 * q[65536] = -q[0]; the table is made exactly antisymmetric. */
void synth_build_table(double* q) {
  const uint32_t n = SYNTH_TABLE_CELLS;
  q[n / 2] = 0.0;
#pragma omp parallel for schedule(dynamic, 256)
  for (int64_t j = 1; j < (int64_t)(n / 2); ++j) {
    double v = std_normal_quantile_lower((double)j / (double)n);
    q[j] = v;
    q[n - j] = -v;
  }
  q[0] = std_normal_quantile_lower(0x1p-20);
  q[n] = -q[0];
}

/* dtype 0: fp32 output (float*), dtype 1: bf16 bits (uint16_t*).
 * Fills out[i] for i in [0, n) with element (offset + i) of tensor
 * (seed, tensor_id), scaled by sigma. */
void synth_fill_host(void* out, int dtype, uint64_t n, uint64_t offset, uint64_t seed,
                     uint32_t tensor_id, double sigma, const double* q) {
  const uint64_t key = synth_stream_key(seed, tensor_id);
  if (dtype == 0) {
    float* o = (float*)out;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
      double z = synth_normal(q, synth_bits(key, offset + (uint64_t)i));
      o[i] = synth_scale_f32(z, sigma);
    }
  } else {
    uint16_t* o = (uint16_t*)out;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
      double z = synth_normal(q, synth_bits(key, offset + (uint64_t)i));
      o[i] = synth_f32_to_bf16(synth_scale_f32(z, sigma));
    }
  }
}

/* Strided variant: fills rows [row0, row0 + nrows) of a row-major
 * [*, ncols] tensor whose element (r, c) is flat index base + r*ncols + c,
 * writing them contiguously into out. Used to build a token subset of x. */
void synth_fill_rows_host(void* out, int dtype, const int64_t* rows, int64_t nrows, int64_t ncols,
                          uint64_t base, uint64_t seed, uint32_t tensor_id, double sigma,
                          const double* q) {
  const uint64_t key = synth_stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    for (int64_t c = 0; c < ncols; ++c) {
      uint64_t idx = base + (uint64_t)rows[r] * (uint64_t)ncols + (uint64_t)c;
      double z = synth_normal(q, synth_bits(key, idx));
      float v = synth_scale_f32(z, sigma);
      if (dtype == 0) ((float*)out)[r * ncols + c] = v;
      else ((uint16_t*)out)[r * ncols + c] = synth_f32_to_bf16(v);
    }
  }
}
