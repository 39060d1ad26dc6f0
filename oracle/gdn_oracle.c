/*
 * Float64 reference for the Gated DeltaNet prefill -- TEST INFRASTRUCTURE.
 *
 * Only the test suite, the package smoke check and the CPU-baseline leg of
 * the benchmark may load this file's library.  The product path never does.
 * It shares no code with the HIP library.
 *
 * What it computes (the plain definition, one token at a time):
 *   The gated delta rule, written for a state H of shape d_k x d_v (the
 *   transpose of the d_v x d_k form S_t = alpha_t S_{t-1} (I - b k k^T) +
 *   b v k^T, o_t = S_t q):
 *
 *       q^ = q / sqrt(sum q^2 + eps),   k^ = k / sqrt(sum k^2 + eps)
 *       alpha = exp(g),                  b = beta (already in [0, 1])
 *       H_t  = alpha * (I - b k^ k^T) H_{t-1} + b k^ v^T
 *       o_t  = scale * H_t^T q^
 *
 *   The serving pages ("Cua-S1 4B 0.2 native text worker"; "Open-Jev-27B-v1.1
 *   native text worker", section "Validation and optimization scope") test
 *   their chunked Gated DeltaNet prefill against float64 references; this is
 *   such a reference.
 *
 *   (I - b k^ k^T) H is expanded as H - b k^ (k^T H); nothing else is
 *   rearranged.  Every product is taken in double precision; inputs arrive
 *   as float (bf16 and fp32 values are exact in float).
 *
 * Layout (all contiguous, last index fastest):
 *   q, k [T, Hk, dk]; v [T, Hv, dv]; g, beta [T, Hv];
 *   cu_seqlens int32 [N+1] (cu[0] = 0, cu[N] = T, non-decreasing);
 *   init_state float [N, Hv, dk, dv] or NULL (= zeros);
 *   out double [T, Hv, dv]; final_state double [N, Hv, dk, dv] or NULL.
 *   Value head h reads key head h / (Hv / Hk).
 *
 * Pins (tests/test_oracle_*.py): closed forms for beta = 0 (pure decay),
 * orthonormal keys (gated linear attention), beta = 1 overwrite, a
 * hand-derived two-token example, explicit d_k x d_k transition products for
 * T <= 8, chunk-size invariance of an independent chunked evaluator,
 * linearity, split/continuation, packing and head grouping.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
  const float *q, *k, *v, *g, *beta, *init;
  const int32_t* cu;
  double *out, *final_state;
  int32_t n_seq, t_tot, hk, hv, dk, dv;
  double scale, eps;
  int64_t n_units;          /* n_seq * hv */
  int64_t next;             /* shared work counter, guarded by lock */
  pthread_mutex_t lock;
} job_t;

/* One (sequence, value head) unit: the token loop. */
static void run_unit(const job_t* J, int64_t unit, double* H, double* qh,
                     double* kh, double* kTH) {
  const int32_t seq = (int32_t)(unit / J->hv);
  const int32_t h = (int32_t)(unit % J->hv);
  const int32_t group = J->hv / J->hk;
  const int32_t kv = h / group; /* key head read by value head h */
  const int32_t dk = J->dk, dv = J->dv;
  const size_t hsz = (size_t)dk * dv;

  if (J->init) {
    const float* s = J->init + ((size_t)seq * J->hv + h) * hsz;
    for (size_t e = 0; e < hsz; ++e) H[e] = (double)s[e];
  } else {
    memset(H, 0, hsz * sizeof(double));
  }

  for (int32_t t = J->cu[seq]; t < J->cu[seq + 1]; ++t) {
    const float* qt = J->q + ((size_t)t * J->hk + kv) * dk;
    const float* kt = J->k + ((size_t)t * J->hk + kv) * dk;
    const float* vt = J->v + ((size_t)t * J->hv + h) * dv;
    double qq = 0.0, kk = 0.0;
    for (int32_t i = 0; i < dk; ++i) {
      qq += (double)qt[i] * (double)qt[i];
      kk += (double)kt[i] * (double)kt[i];
    }
    const double rq = 1.0 / sqrt(qq + J->eps);
    const double rk = 1.0 / sqrt(kk + J->eps);
    for (int32_t i = 0; i < dk; ++i) {
      qh[i] = (double)qt[i] * rq;
      kh[i] = (double)kt[i] * rk;
    }
    const double alpha = exp((double)J->g[(size_t)t * J->hv + h]);
    const double b = (double)J->beta[(size_t)t * J->hv + h];

    /* kTH = k^T H  (a row of length dv) */
    for (int32_t j = 0; j < dv; ++j) kTH[j] = 0.0;
    for (int32_t i = 0; i < dk; ++i)
      for (int32_t j = 0; j < dv; ++j) kTH[j] += kh[i] * H[(size_t)i * dv + j];

    /* H = alpha * (H - b k^ (k^T H)) + b k^ v^T */
    for (int32_t i = 0; i < dk; ++i)
      for (int32_t j = 0; j < dv; ++j) {
        double* hij = &H[(size_t)i * dv + j];
        *hij = alpha * (*hij - b * kh[i] * kTH[j]) + b * kh[i] * (double)vt[j];
      }

    /* o = scale * H^T q^ */
    double* ot = J->out + ((size_t)t * J->hv + h) * dv;
    for (int32_t j = 0; j < dv; ++j) {
      double acc = 0.0;
      for (int32_t i = 0; i < dk; ++i) acc += H[(size_t)i * dv + j] * qh[i];
      ot[j] = J->scale * acc;
    }
  }

  if (J->final_state) {
    double* f = J->final_state + ((size_t)seq * J->hv + h) * hsz;
    memcpy(f, H, hsz * sizeof(double));
  }
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  const size_t hsz = (size_t)J->dk * J->dv;
  double* H = (double*)malloc(hsz * sizeof(double));
  double* qh = (double*)malloc((size_t)J->dk * sizeof(double));
  double* kh = (double*)malloc((size_t)J->dk * sizeof(double));
  double* kTH = (double*)malloc((size_t)J->dv * sizeof(double));
  if (H && qh && kh && kTH) {
    for (;;) {
      pthread_mutex_lock(&J->lock);
      const int64_t u = J->next++;
      pthread_mutex_unlock(&J->lock);
      if (u >= J->n_units) break;
      run_unit(J, u, H, qh, kh, kTH);
    }
  }
  free(H);
  free(qh);
  free(kh);
  free(kTH);
  return NULL;
}

/* Returns 0 on success, -1 on bad arguments (nothing is written).
 * n_threads <= 0 uses the number of online processors. */
int gdn_oracle_f64(const float* q, const float* k, const float* v,
                   const float* g, const float* beta, const int32_t* cu,
                   int32_t n_seq, const float* init_state, double* out,
                   double* final_state, int32_t t_tot, int32_t hk, int32_t hv,
                   int32_t dk, int32_t dv, double scale, double eps,
                   int32_t n_threads) {
  if (!q || !k || !v || !g || !beta || !cu || !out) return -1;
  if (n_seq < 0 || t_tot < 0 || hk <= 0 || hv <= 0 || dk <= 0 || dv <= 0) return -1;
  if (hv % hk) return -1;
  if (cu[0] != 0 || cu[n_seq] != t_tot) return -1;
  for (int32_t i = 0; i < n_seq; ++i)
    if (cu[i + 1] < cu[i]) return -1;

  job_t J;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.init = init_state;
  J.cu = cu; J.out = out; J.final_state = final_state;
  J.n_seq = n_seq; J.t_tot = t_tot; J.hk = hk; J.hv = hv; J.dk = dk; J.dv = dv;
  J.scale = scale; J.eps = eps;
  J.n_units = (int64_t)n_seq * hv;
  J.next = 0;
  pthread_mutex_init(&J.lock, NULL);

  if (n_threads <= 0) n_threads = (int32_t)sysconf(_SC_NPROCESSORS_ONLN);
  if (n_threads < 1) n_threads = 1;
  if (n_threads > J.n_units) n_threads = (int32_t)(J.n_units > 0 ? J.n_units : 1);

  /* Threads only share out whole units; if none can be started the
   * calling thread does all the work itself. */
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)n_threads);
  int started = 0;
  if (th)
    for (int32_t i = 0; i < n_threads; ++i) {
      if (pthread_create(&th[i], NULL, worker, &J) != 0) break;
      ++started;
    }
  if (started == 0) worker(&J);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.lock);
  return 0;
}
