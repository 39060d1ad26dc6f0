/* Drives the float64 oracle (oracle/gdn_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer on the CPU: packed batches with empty and
 * one-token sequences, grouped heads, an initial state aliased by the final
 * state, several thread counts, and the argument checks.  Exit status 0
 * means every call returned the expected status and every output is finite;
 * a sanitizer report aborts the run. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gdn_oracle_f64(const float* q, const float* k, const float* v, const float* g,
                   const float* beta, const int32_t* cu, int32_t n_seq, const float* init_state,
                   double* out, double* final_state, int32_t t_tot, int32_t hk, int32_t hv,
                   int32_t dk, int32_t dv, double scale, double eps, int32_t n_threads);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static float uniform(void) { /* xorshift64*, in [-1, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (float)((rng_state * 0x2545F4914F6CDD1Dull) >> 40) / (float)(1u << 23) - 1.0f;
}

static float* fill(size_t n, float lo, float hi) {
  float* p = (float*)malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5f * (uniform() + 1.0f);
  return p;
}

static int finite_all(const double* p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static int run_case(int n_seq, const int32_t* lens, int hk, int hv, int dk, int dv, int with_init,
                    int alias, int threads) {
  int32_t* cu = (int32_t*)malloc((size_t)(n_seq + 1) * sizeof(int32_t));
  cu[0] = 0;
  for (int i = 0; i < n_seq; ++i) cu[i + 1] = cu[i] + lens[i];
  const int T = cu[n_seq];
  float* q = fill((size_t)T * hk * dk, -1, 1);
  float* k = fill((size_t)T * hk * dk, -1, 1);
  float* v = fill((size_t)T * hv * dv, -1, 1);
  float* g = fill((size_t)T * hv, -3, 0);
  float* b = fill((size_t)T * hv, 0, 1);
  const size_t ssz = (size_t)n_seq * hv * dk * dv;
  float* init = with_init ? fill(ssz, -0.5f, 0.5f) : NULL;
  double* out = (double*)malloc(((size_t)T * hv * dv + 1) * sizeof(double));
  double* fin = (double*)malloc((ssz + 1) * sizeof(double));
  int ok = 1;
  if (alias && init) {
    /* the final state written over a double copy of the initial one */
    for (size_t i = 0; i < ssz; ++i) fin[i] = init[i];
  }
  const int rc = gdn_oracle_f64(q, k, v, g, b, cu, n_seq, init, out, fin, T, hk, hv, dk, dv, 0.5,
                                1e-6, threads);
  if (rc != 0) ok = 0;
  if (!finite_all(out, (size_t)T * hv * dv) || !finite_all(fin, ssz)) ok = 0;
  free(cu); free(q); free(k); free(v); free(g); free(b); free(init); free(out); free(fin);
  return ok;
}

int main(void) {
  int fails = 0;
  const int32_t l1[] = {0, 1, 7, 0, 33, 2, 0};
  fails += !run_case(7, l1, 2, 4, 16, 8, 1, 0, 1);
  fails += !run_case(7, l1, 1, 3, 8, 16, 0, 0, 3);
  const int32_t l2[] = {64, 65};
  fails += !run_case(2, l2, 2, 2, 32, 32, 1, 1, 2);
  const int32_t l3[] = {0};
  fails += !run_case(1, l3, 1, 1, 4, 4, 1, 0, 1);
  /* argument checks: each call returns -1 and touches nothing */
  float x[16] = {0};
  double o[16];
  int32_t bad_cu[3] = {0, 2, 1};
  int32_t good_cu[2] = {0, 1};
  if (gdn_oracle_f64(x, x, x, x, x, bad_cu, 2, NULL, o, NULL, 1, 1, 1, 2, 2, 1, 0, 1) != -1) ++fails;
  if (gdn_oracle_f64(x, x, x, x, x, good_cu, 1, NULL, o, NULL, 1, 2, 3, 2, 2, 1, 0, 1) != -1) ++fails;
  if (gdn_oracle_f64(NULL, x, x, x, x, good_cu, 1, NULL, o, NULL, 1, 1, 1, 2, 2, 1, 0, 1) != -1) ++fails;
  if (gdn_oracle_f64(x, x, x, x, x, good_cu, 1, NULL, o, NULL, 2, 1, 1, 2, 2, 1, 0, 1) != -1) ++fails;
  printf("oracle under sanitizers: %d failure(s)\n", fails);
  return fails ? 1 : 0;
}
