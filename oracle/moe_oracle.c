/*
 * CPU oracle for the forward pass of one sparse Mixture-of-Experts block.
 *
 * TEST INFRASTRUCTURE ONLY: this file is used by the test suite, by the
 * smoke check and by the benchmark's CPU-baseline leg. The product path never
 * links, loads or calls it, and it shares no code with the GPU library.
 *
 * It is the plain definition, written out token by token, with every sum
 * accumulated in double:
 *
 *   router  (the router maps the token's embedding to one score per expert --
 *            Qwen3.6 MoE explorer page, section on the MoE router):
 *              l_e = fp32( sum_i x_i * W_r[i, e]  (+ b_e) )
 *   top-k   (same section: a probability for each expert, the K most
 *            probable kept): S = the k largest l_e, ties to the lower index,
 *            listed by descending logit; gap = l_(k) - l_(k+1) (+inf if k = E)
 *   softmax p_e = exp(l_e - max l) / sum_e' exp(l_e' - max l) over all E;
 *           w_j = p_j / sum_{i in S} p_i when renormalising, else w_j = p_j
 *   experts (hidden_act "silu", moe_intermediate_size -- the Qwen3.8-Max
 *            architecture page, config.json listing; three d x I matrices per
 *            expert with no biases, as the per-block parameter count on the
 *            overview page's parameter table implies):
 *              y_j = (silu(x W_g[j]) * (x W_u[j])) W_d[j],  silu(z) = z / (1 + e^-z)
 *   shared  one always-active expert (MoE explorer page, router section; the
 *           Qwen3-Next article) of size shared_expert_intermediate_size, added
 *           with no weight:  s = (silu(x W_gs) * (x W_us)) W_ds
 *   output  out = sum_{j in S} w_j y_j + s
 *
 * Readings where the pages are silent: softmax over all E then top-k (equal
 * to a softmax over the k kept logits when renormalising); selection on the
 * fp32 logits; lower index wins ties; the shared expert is unweighted.
 *
 * Around the block (moe_oracle_rmsnorm; the residual add is done by the
 * caller): zero-centred RMSNorm in front of it -- the Qwen3-Next article names
 * Zero-Centered RMSNorm, whose parameters start at zero, so the scale is
 * 1 + gamma; the configuration listing on the Qwen3.8-Max architecture page
 * gives rms_norm_eps = 1e-6:
 *              h = x / sqrt(mean_i x_i^2 + eps) * (1 + gamma)
 * and the layer's output is x + MoE(h). The parameter table of the overview
 * page counts two norms per layer plus a final one, which places a norm in
 * front of every MoE block.
 *
 * Element types: x and the expert weights are fp32 (dtype 0) or bf16 bit
 * patterns (dtype 1, widened exactly); the router weight and bias are fp32.
 * Expert weights are passed as one pointer per expert so that a caller may
 * supply only the experts the given tokens select (NULL for the others).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };
enum { ORACLE_OK = 0, ORACLE_ERR_ARG = -1, ORACLE_ERR_MISSING_EXPERT = -2, ORACLE_ERR_NOMEM = -3 };

/* element i of an fp32 or bf16 array, widened to double */
static double elem(const void* p, int dtype, size_t i) {
  if (dtype == ORACLE_F32) return (double)((const float*)p)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* row r of a [rows, n] matrix, widened to double */
static void widen_row(double* dst, const void* m, int dtype, size_t r, size_t n) {
  for (size_t c = 0; c < n; ++c) dst[c] = elem(m, dtype, r * n + c);
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* y[0..d) = (silu(x W_g) * (x W_u)) W_d for one token x[0..d);
 * W_g, W_u are [d, n], W_d is [n, d]; tmp holds 3*n + max(n, d) doubles. */
static void swiglu_ffn(const double* x, int32_t d, int32_t n, int dtype, const void* wg, const void* wu,
                       const void* wd, double* y, double* tmp) {
  double* g = tmp;
  double* u = tmp + n;
  double* h = tmp + 2 * (size_t)n;
  double* row = tmp + 3 * (size_t)n; /* caller sizes tmp as 3*n + max(n, d) */
  for (int32_t i = 0; i < n; ++i) g[i] = u[i] = 0.0;
  for (int32_t c = 0; c < d; ++c) {
    widen_row(row, wg, dtype, (size_t)c, (size_t)n);
    for (int32_t i = 0; i < n; ++i) g[i] += x[c] * row[i];
    widen_row(row, wu, dtype, (size_t)c, (size_t)n);
    for (int32_t i = 0; i < n; ++i) u[i] += x[c] * row[i];
  }
  for (int32_t i = 0; i < n; ++i) h[i] = silu(g[i]) * u[i];
  for (int32_t c = 0; c < d; ++c) y[c] = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    widen_row(row, wd, dtype, (size_t)i, (size_t)d);
    for (int32_t c = 0; c < d; ++c) y[c] += h[i] * row[c];
  }
}

/* Router, top-k and softmax weights for one token.
 * logits[E] (fp32), idx[k], w[k], *gap are written. */
static void route_token(const double* x, int32_t d, int32_t E, int32_t k, int32_t renorm,
                        const float* w_router, const float* bias, float* logits, int32_t* idx, double* w,
                        double* gap, double* acc, char* taken) {
  for (int32_t e = 0; e < E; ++e) acc[e] = 0.0;
  for (int32_t c = 0; c < d; ++c)
    for (int32_t e = 0; e < E; ++e) acc[e] += x[c] * (double)w_router[(size_t)c * E + e];
  for (int32_t e = 0; e < E; ++e) {
    double v = acc[e];
    if (bias) v += (double)bias[e];
    logits[e] = (float)v; /* rounded once to fp32 */
  }

  /* top-k by repeated selection of the largest unselected logit; a strict '>'
   * scanning upwards keeps the lowest index among equal values */
  memset(taken, 0, (size_t)E);
  for (int32_t j = 0; j < k; ++j) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e)
      if (!taken[e] && (best < 0 || logits[e] > logits[best])) best = e;
    idx[j] = best;
    taken[best] = 1;
  }
  if (k < E) {
    int32_t next = -1;
    for (int32_t e = 0; e < E; ++e)
      if (!taken[e] && (next < 0 || logits[e] > logits[next])) next = e;
    *gap = (double)logits[idx[k - 1]] - (double)logits[next];
  } else {
    *gap = INFINITY;
  }

  /* softmax over all E experts, in double */
  double m = (double)logits[idx[0]];
  double z = 0.0;
  for (int32_t e = 0; e < E; ++e) z += exp((double)logits[e] - m);
  double sel = 0.0;
  for (int32_t j = 0; j < k; ++j) {
    w[j] = exp((double)logits[idx[j]] - m) / z;
    sel += w[j];
  }
  if (renorm)
    for (int32_t j = 0; j < k; ++j) w[j] /= sel;
}

static int check_dims(int64_t T, int32_t d, int32_t E, int32_t k) {
  if (T < 0 || d <= 0 || E <= 0 || k <= 0 || k > E) return ORACLE_ERR_ARG;
  return ORACLE_OK;
}

/* Router + top-k only. x: [T, d] (dtype), w_router: [d, E] fp32, bias: [E] or NULL.
 * Outputs (each optional except topk_idx): logits [T, E] fp32, topk_idx [T, k], topk_w [T, k],
 * gap [T]. */
int moe_oracle_router(int64_t T, int32_t d, int32_t E, int32_t k, int32_t renorm, int32_t dtype,
                      const void* x, const float* w_router, const float* bias, float* logits_out,
                      int32_t* topk_idx, double* topk_w, double* gap_out) {
  int rc = check_dims(T, d, E, k);
  if (rc) return rc;
  if (!x || !w_router || !topk_idx) return ORACLE_ERR_ARG;
  int err = 0;
#pragma omp parallel
  {
    double* xr = (double*)malloc(sizeof(double) * (size_t)d);
    double* acc = (double*)malloc(sizeof(double) * (size_t)E);
    char* taken = (char*)malloc((size_t)E);
    float* lg = (float*)malloc(sizeof(float) * (size_t)E);
    double* w = (double*)malloc(sizeof(double) * (size_t)k);
    const int ok = xr && acc && taken && lg && w;
    if (!ok) {
#pragma omp atomic write
      err = 1;
    }
    /* every thread reaches the worksharing loop; one without buffers skips its tokens */
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
      if (!ok) continue;
      double gap;
      widen_row(xr, x, dtype, (size_t)t, (size_t)d);
      route_token(xr, d, E, k, renorm, w_router, bias, lg, topk_idx + t * k, w, &gap, acc, taken);
      if (logits_out) memcpy(logits_out + t * E, lg, sizeof(float) * (size_t)E);
      if (topk_w) memcpy(topk_w + t * k, w, sizeof(double) * (size_t)k);
      if (gap_out) gap_out[t] = gap;
    }
    free(xr); free(acc); free(taken); free(lg); free(w);
  }
  return err ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/* Whole block. x: [T, d]; w_router [d, E] fp32; bias [E] or NULL; wg[e], wu[e]: [d, I] and
 * wd[e]: [I, d] per expert (NULL allowed for experts no token selects); wg_s, wu_s [d, Is],
 * wd_s [Is, d] (ignored when Is == 0). out: [T, d] double. topk_idx / topk_w / gap optional. */
int moe_oracle_forward(int64_t T, int32_t d, int32_t E, int32_t k, int32_t I, int32_t Is, int32_t renorm,
                       int32_t dtype, const void* x, const float* w_router, const float* bias,
                       const void* const* wg, const void* const* wu, const void* const* wd,
                       const void* wg_s, const void* wu_s, const void* wd_s, double* out,
                       int32_t* topk_idx, double* topk_w, double* gap_out) {
  int rc = check_dims(T, d, E, k);
  if (rc) return rc;
  if (I <= 0 || Is < 0 || !x || !w_router || !wg || !wu || !wd || !out) return ORACLE_ERR_ARG;
  if (Is > 0 && (!wg_s || !wu_s || !wd_s)) return ORACLE_ERR_ARG;
  int err = 0;
  const int32_t nmax = I > Is ? I : Is;
  const int32_t rowlen = nmax > d ? nmax : d;
#pragma omp parallel
  {
    double* xr = (double*)malloc(sizeof(double) * (size_t)d);
    double* acc = (double*)malloc(sizeof(double) * (size_t)E);
    char* taken = (char*)malloc((size_t)E);
    float* lg = (float*)malloc(sizeof(float) * (size_t)E);
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    double* w = (double*)malloc(sizeof(double) * (size_t)k);
    double* y = (double*)malloc(sizeof(double) * (size_t)d);
    double* tmp = (double*)malloc(sizeof(double) * (3 * (size_t)nmax + (size_t)rowlen));
    const int ok = xr && acc && taken && lg && idx && w && y && tmp;
    if (!ok) {
#pragma omp atomic write
      err = ORACLE_ERR_NOMEM;
    }
    /* every thread reaches the worksharing loop; one without buffers skips its tokens */
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
      if (!ok) continue;
      double gap;
      double* o = out + t * d;
      widen_row(xr, x, dtype, (size_t)t, (size_t)d);
      route_token(xr, d, E, k, renorm, w_router, bias, lg, idx, w, &gap, acc, taken);
      for (int32_t c = 0; c < d; ++c) o[c] = 0.0;
      for (int32_t j = 0; j < k; ++j) {
        int32_t e = idx[j];
        if (!wg[e] || !wu[e] || !wd[e]) {
#pragma omp atomic write
          err = ORACLE_ERR_MISSING_EXPERT;
          break;
        }
        swiglu_ffn(xr, d, I, dtype, wg[e], wu[e], wd[e], y, tmp);
        for (int32_t c = 0; c < d; ++c) o[c] += w[j] * y[c];
      }
      if (Is > 0) {
        swiglu_ffn(xr, d, Is, dtype, wg_s, wu_s, wd_s, y, tmp);
        for (int32_t c = 0; c < d; ++c) o[c] += y[c];
      }
      if (topk_idx) memcpy(topk_idx + t * k, idx, sizeof(int32_t) * (size_t)k);
      if (topk_w) memcpy(topk_w + t * k, w, sizeof(double) * (size_t)k);
      if (gap_out) gap_out[t] = gap;
    }
    free(xr); free(acc); free(taken); free(lg); free(idx); free(w); free(y); free(tmp);
  }
  return err;
}

/* One expert's output for a list of (token row, expert) pairs: for pair p,
 *   y[p] = (silu(x_r W_g) * (x_r W_u)) W_d  with r = rows[p] and the pair's own
 * expert matrices wg[p], wu[p] ([d, n]) and wd[p] ([n, d]) -- the expert of the
 * header, token by token, with no weighting. y: [npairs, d] double. The caller
 * forms the weighted sums; this lets it visit the experts a few at a time when
 * all of their weights do not fit in host memory at once. */
int moe_oracle_expert_rows(int64_t npairs, int32_t d, int32_t n, int32_t dtype, const void* x, const int64_t* rows,
                           const void* const* wg, const void* const* wu, const void* const* wd, double* y) {
  if (npairs < 0 || d <= 0 || n <= 0 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16)) return ORACLE_ERR_ARG;
  if (npairs > 0 && (!x || !rows || !wg || !wu || !wd || !y)) return ORACLE_ERR_ARG;
  int err = 0;
  const int32_t rowlen = n > d ? n : d;
#pragma omp parallel
  {
    double* xr = (double*)malloc(sizeof(double) * (size_t)d);
    double* tmp = (double*)malloc(sizeof(double) * (3 * (size_t)n + (size_t)rowlen));
    const int ok = xr && tmp;
    if (!ok) {
#pragma omp atomic write
      err = ORACLE_ERR_NOMEM;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t p = 0; p < npairs; ++p) {
      if (!ok) continue;
      if (!wg[p] || !wu[p] || !wd[p] || rows[p] < 0) {
#pragma omp atomic write
        err = ORACLE_ERR_ARG;
        continue;
      }
      widen_row(xr, x, dtype, (size_t)rows[p], (size_t)d);
      swiglu_ffn(xr, d, n, dtype, wg[p], wu[p], wd[p], y + p * d, tmp);
    }
    free(xr);
    free(tmp);
  }
  return err;
}

/* v rounded to bf16, round to nearest with ties to even, from the exact double
 * (not through fp32): significand scaled to [128, 256), rounded by rint in the
 * default rounding mode, scaled back. Normal range only (|v| >= 2^-126 or 0). */
static uint16_t round_bf16(double v) {
  if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
  int e;
  const double m = frexp(v, &e); /* v = m 2^e, 0.5 <= |m| < 1 */
  const double r = ldexp(rint(ldexp(m, 8)), e - 8);
  const float f = (float)r; /* exact: 8 significant bits */
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  return (uint16_t)(bits >> 16);
}

/* Zero-centred RMSNorm of each of the T rows of x [T, d] (see the header):
 *   h = x / sqrt(mean(x^2) + eps) * (1 + gamma), in double,
 * stored in the element type of x (rounded once: bf16 by round_bf16, fp32 by
 * the conversion). gamma [d] has the element type of x. */
int moe_oracle_rmsnorm(int64_t T, int32_t d, int32_t dtype, const void* x, const void* gamma, double eps, void* h) {
  if (T < 0 || d < 1 || (dtype != ORACLE_F32 && dtype != ORACLE_BF16) || !(eps >= 0.0)) return ORACLE_ERR_ARG;
  if (T > 0 && (!x || !gamma || !h)) return ORACLE_ERR_ARG;
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int32_t i = 0; i < d; ++i) {
      const double v = elem(x, dtype, (size_t)t * d + i);
      ss += v * v;
    }
    const double inv = 1.0 / sqrt(ss / d + eps);
    for (int32_t i = 0; i < d; ++i) {
      const double v = elem(x, dtype, (size_t)t * d + i) * inv * (1.0 + elem(gamma, dtype, (size_t)i));
      if (dtype == ORACLE_F32)
        ((float*)h)[(size_t)t * d + i] = (float)v;
      else
        ((uint16_t*)h)[(size_t)t * d + i] = round_bf16(v);
    }
  }
  return ORACLE_OK;
}

/* Threads the parallel regions above use (OpenMP's current maximum). */
int moe_oracle_threads(void) { return omp_get_max_threads(); }
