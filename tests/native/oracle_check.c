/* Runs every entry point of the CPU oracle (oracle/moe_oracle.c) on small random inputs under the
 * host sanitizers (AddressSanitizer, UndefinedBehaviorSanitizer), built by the CPU test suite with
 * gcc. Beyond memory safety it checks what holds for any input: return codes, k distinct indices
 * in range per token, routing weights summing to one with renormalisation, finite outputs, and
 * the error codes of bad calls. Exit status 0 and a last line "oracle_check ok" mean all held. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int moe_oracle_router(int64_t T, int32_t d, int32_t E, int32_t k, int32_t renorm, int32_t dtype, const void* x,
                      const float* w_router, const float* bias, float* logits_out, int32_t* topk_idx, double* topk_w,
                      double* gap_out);
int moe_oracle_forward(int64_t T, int32_t d, int32_t E, int32_t k, int32_t I, int32_t Is, int32_t renorm,
                       int32_t dtype, const void* x, const float* w_router, const float* bias,
                       const void* const* wg, const void* const* wu, const void* const* wd, const void* wg_s,
                       const void* wu_s, const void* wd_s, double* out, int32_t* topk_idx, double* topk_w,
                       double* gap_out);
int moe_oracle_expert_rows(int64_t npairs, int32_t d, int32_t n, int32_t dtype, const void* x, const int64_t* rows,
                           const void* const* wg, const void* const* wu, const void* const* wd, double* y);
int moe_oracle_rmsnorm(int64_t T, int32_t d, int32_t dtype, const void* x, const void* gamma, double eps, void* h);
int moe_oracle_threads(void);

static int failures = 0;
#define CHECK(cond, ...)            \
  do {                              \
    if (!(cond)) {                  \
      ++failures;                   \
      fprintf(stderr, "FAIL: ");    \
      fprintf(stderr, __VA_ARGS__); \
      fprintf(stderr, "\n");        \
    }                               \
  } while (0)

static uint64_t rng_state = 88172645463325252ull;
static double urand(void) { /* xorshift64, uniform in [-1, 1) */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (double)(rng_state >> 11) / (double)(1ull << 52) - 1.0;
}

/* n random values as fp32 (dtype 0) or as bf16 bit patterns by truncation (dtype 1) */
static void* rand_array(size_t n, int dtype, double scale) {
  void* p = malloc(n * (dtype ? 2 : 4) + 1);
  for (size_t i = 0; i < n; ++i) {
    float f = (float)(urand() * scale);
    if (dtype) {
      uint32_t b;
      memcpy(&b, &f, 4);
      ((uint16_t*)p)[i] = (uint16_t)(b >> 16);
    } else {
      ((float*)p)[i] = f;
    }
  }
  return p;
}

static void run_case(int64_t T, int d, int E, int k, int I, int Is, int renorm, int dtype, int with_bias) {
  void* x = rand_array((size_t)T * d, dtype, 2.0);
  float* wr = (float*)rand_array((size_t)d * E, 0, 1.0);
  float* bias = with_bias ? (float*)rand_array((size_t)E, 0, 0.5) : NULL;
  const void** wg = calloc((size_t)E, sizeof(void*));
  const void** wu = calloc((size_t)E, sizeof(void*));
  const void** wd = calloc((size_t)E, sizeof(void*));
  for (int e = 0; e < E; ++e) {
    wg[e] = rand_array((size_t)d * I, dtype, 0.3);
    wu[e] = rand_array((size_t)d * I, dtype, 0.3);
    wd[e] = rand_array((size_t)I * d, dtype, 0.3);
  }
  void* gs = Is ? rand_array((size_t)d * Is, dtype, 0.3) : NULL;
  void* us = Is ? rand_array((size_t)d * Is, dtype, 0.3) : NULL;
  void* ds = Is ? rand_array((size_t)Is * d, dtype, 0.3) : NULL;
  double* out = malloc(sizeof(double) * (size_t)(T * d + 1));
  int32_t* idx = malloc(sizeof(int32_t) * (size_t)(T * k + 1));
  double* w = malloc(sizeof(double) * (size_t)(T * k + 1));
  double* gap = malloc(sizeof(double) * (size_t)(T + 1));
  float* logits = malloc(sizeof(float) * (size_t)(T * E + 1));

  int rc = moe_oracle_forward(T, d, E, k, I, Is, renorm, dtype, x, wr, bias, wg, wu, wd, gs, us, ds, out, idx, w, gap);
  CHECK(rc == 0, "forward rc %d (T=%lld d=%d E=%d k=%d)", rc, (long long)T, d, E, k);
  for (int64_t t = 0; t < T; ++t) {
    double s = 0.0;
    for (int j = 0; j < k; ++j) {
      const int32_t e = idx[t * k + j];
      CHECK(e >= 0 && e < E, "index %d out of range", e);
      for (int j2 = 0; j2 < j; ++j2) CHECK(idx[t * k + j2] != e, "repeated expert %d", e);
      s += w[t * k + j];
    }
    if (renorm) CHECK(fabs(s - 1.0) < 1e-12, "weights sum to %.17g", s);
    CHECK(k < E ? gap[t] >= 0.0 : isinf(gap[t]), "gap %g", gap[t]);
    for (int c = 0; c < d; ++c) CHECK(isfinite(out[t * d + c]), "non-finite output");
  }
  rc = moe_oracle_router(T, d, E, k, renorm, dtype, x, wr, bias, logits, idx, w, gap);
  CHECK(rc == 0, "router rc %d", rc);
  /* per-pair experts: every token with expert (t mod E) */
  if (T > 0) {
    int64_t* rows = malloc(sizeof(int64_t) * (size_t)T);
    const void** pg = malloc(sizeof(void*) * (size_t)T);
    const void** pu = malloc(sizeof(void*) * (size_t)T);
    const void** pd = malloc(sizeof(void*) * (size_t)T);
    double* y = malloc(sizeof(double) * (size_t)(T * d));
    for (int64_t t = 0; t < T; ++t) {
      rows[t] = T - 1 - t;
      pg[t] = wg[t % E];
      pu[t] = wu[t % E];
      pd[t] = wd[t % E];
    }
    rc = moe_oracle_expert_rows(T, d, I, dtype, x, rows, pg, pu, pd, y);
    CHECK(rc == 0, "expert_rows rc %d", rc);
    rows[0] = -1;
    CHECK(moe_oracle_expert_rows(T, d, I, dtype, x, rows, pg, pu, pd, y) != 0, "negative row accepted");
    free(rows); free(pg); free(pu); free(pd); free(y);
  }
  /* a selected expert missing -> error code, no crash */
  if (T > 0) {
    const void* keep = wg[idx[0]];
    wg[idx[0]] = NULL;
    rc = moe_oracle_forward(T, d, E, k, I, Is, renorm, dtype, x, wr, bias, wg, wu, wd, gs, us, ds, out, NULL, NULL,
                            NULL);
    CHECK(rc != 0, "missing expert not reported");
    wg[idx[0]] = keep;
  }
  /* the norm on the same rows */
  if (T > 0) {
    void* gamma = rand_array((size_t)d, dtype, 0.1);
    void* h = malloc((size_t)T * d * (dtype ? 2 : 4));
    CHECK(moe_oracle_rmsnorm(T, d, dtype, x, gamma, 1e-6, h) == 0, "rmsnorm rc");
    CHECK(moe_oracle_rmsnorm(T, d, dtype, x, gamma, -1.0, h) != 0, "negative eps accepted");
    free(gamma); free(h);
  }
  for (int e = 0; e < E; ++e) {
    free((void*)wg[e]); free((void*)wu[e]); free((void*)wd[e]);
  }
  free(wg); free(wu); free(wd); free(gs); free(us); free(ds);
  free(x); free(wr); free(bias); free(out); free(idx); free(w); free(gap); free(logits);
}

int main(void) {
  /* T, d, E, k, I, Is, renorm, dtype, bias */
  run_case(37, 24, 6, 2, 16, 8, 1, 0, 0);
  run_case(37, 24, 6, 2, 16, 8, 0, 1, 1);
  run_case(5, 16, 1, 1, 8, 8, 1, 1, 0);   /* one expert */
  run_case(9, 16, 4, 4, 8, 0, 1, 0, 1);   /* k = E, no shared expert */
  run_case(64, 40, 33, 16, 24, 16, 1, 1, 1);
  run_case(0, 16, 4, 2, 8, 8, 1, 0, 0);   /* no tokens */
  CHECK(moe_oracle_forward(3, 8, 4, 5, 8, 0, 1, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                           NULL, NULL) != 0, "k > E accepted");
  CHECK(moe_oracle_router(3, 8, 4, 2, 1, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL) != 0, "NULL x accepted");
  CHECK(moe_oracle_threads() >= 1, "threads");
  if (failures) {
    fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  printf("oracle_check ok\n");
  return 0;
}
