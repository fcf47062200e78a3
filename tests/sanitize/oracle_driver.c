/*
 * oracle_driver.c -- runs every entry point of oracle/dash_oracle.c on small
 * seeded inputs, valid and invalid, so that a build of the oracle with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py)
 * sees every code path: entmax by sorting and by bisection, summaries with
 * and without a summary query, causal and non-causal forward rows with every
 * optional output, the prefill backward, and the argument checks.
 * Exits 0 when every call returned what it should; the sanitizers abort on
 * any memory or undefined-behaviour error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double oracle_entmax(const double* x, int n, double alpha, int method, double* p);
void oracle_summaries(const float* k, int B, int Hkv, int64_t kv_stride, int d, int bs,
                      int64_t nblocks, const float* w_s, const float* q_bar, double* out);
int oracle_forward_rows(const float* q_rows, const int64_t* row_b, const int64_t* row_pos,
                        int64_t nrows, const float* k, const float* v, int64_t kv_stride,
                        int64_t n_kv, int B, int H, int Hkv, int d, int bs, double alpha,
                        double gamma, double sigma, int window, int causal, const double* summ,
                        int64_t summ_stride, int64_t nb_out, double* o, double* tau,
                        double* x_out, double* p_out, double* pbar, int nthreads);
int oracle_prefill_backward(const float* q, const float* k, const float* v, const float* w_s,
                            const float* d_o, int B, int H, int Hkv, int64_t N, int d, int bs,
                            double alpha, double gamma, double sigma, int window, double* dq,
                            double* dk, double* dv, double* dws, int nthreads);
int oracle_max_threads(void);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) {   /* splitmix64 -> [0, 1) */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}
static float* randf(size_t n, double scale) {
  float* a = (float*)malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) a[i] = (float)((2.0 * uniform() - 1.0) * scale);
  return a;
}
static int failures = 0;
static void expect(int ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}

static void run_entmax(void) {
  const double alphas[] = {1.25, 1.5, 1.7, 2.0};
  const int sizes[] = {1, 7, 100};
  for (int ai = 0; ai < 4; ++ai)
    for (int si = 0; si < 3; ++si)
      for (int method = 0; method < 2; ++method) {
        const int n = sizes[si];
        double* x = (double*)malloc(n * sizeof(double));
        double* p = (double*)malloc(n * sizeof(double));
        for (int j = 0; j < n; ++j) x[j] = j % 3 == 0 ? 0.25 : 2.0 * uniform();   /* with ties */
        const double tau = oracle_entmax(x, n, alphas[ai], method, p);
        double sum = 0.0;
        for (int j = 0; j < n; ++j) sum += p[j];
        expect(isfinite(tau) && fabs(sum - 1.0) < 1e-6, "entmax sums to one");
        free(x);
        free(p);
      }
  double dummy = 0.0;
  expect(isnan(oracle_entmax(&dummy, 0, 1.5, 0, &dummy)), "entmax of nothing is NaN");
}

static void run_summaries(void) {
  const int B = 2, Hkv = 2, L = 256, d = 16, bs = 64, nblocks = 3;
  float* k = randf((size_t)B * Hkv * L * d, 1.0);
  float* w = randf((size_t)d * d, 0.3);
  float* qbar = randf((size_t)Hkv * d, 1.0);
  double* out = (double*)malloc(sizeof(double) * B * Hkv * nblocks * d);
  oracle_summaries(k, B, Hkv, L, d, bs, nblocks, w, NULL, out);
  oracle_summaries(k, B, Hkv, L, d, bs, nblocks, w, qbar, out);
  expect(isfinite(out[B * Hkv * nblocks * d - 1]), "summaries finite");
  free(k);
  free(w);
  free(qbar);
  free(out);
}

static void run_forward(void) {
  const int B = 2, H = 4, Hkv = 2, L = 256, d = 16, bs = 64, nb = L / bs;
  float* k = randf((size_t)B * Hkv * L * d, 1.0);
  float* v = randf((size_t)B * Hkv * L * d, 1.0);
  float* w = randf((size_t)d * d, 0.3);
  double* summ = (double*)malloc(sizeof(double) * B * Hkv * nb * d);
  oracle_summaries(k, B, Hkv, L, d, bs, nb, w, NULL, summ);
  const int64_t nrows = (int64_t)B * L;
  float* q = randf((size_t)nrows * H * d, 2.0);
  int64_t* rb = (int64_t*)malloc(sizeof(int64_t) * nrows);
  int64_t* rp = (int64_t*)malloc(sizeof(int64_t) * nrows);
  for (int64_t r = 0; r < nrows; ++r) {
    rb[r] = r / L;
    rp[r] = r % L;
  }
  double* o = (double*)malloc(sizeof(double) * nrows * H * d);
  double* tau = (double*)malloc(sizeof(double) * nrows * H);
  double* x = (double*)malloc(sizeof(double) * nrows * H * nb);
  double* p = (double*)malloc(sizeof(double) * nrows * H * nb);
  double* pbar = (double*)malloc(sizeof(double) * nrows * Hkv * nb);
  const double alphas[] = {1.25, 1.5, 1.7, 2.0};
  for (int ai = 0; ai < 4; ++ai)
    for (int window = 1; window <= 2; ++window) {
      const int rc = oracle_forward_rows(q, rb, rp, nrows, k, v, L, L, B, H, Hkv, d, bs,
                                         alphas[ai], 4.0, ai % 2 ? 0.5 : 1.0, window, 1, summ,
                                         nb, nb, o, tau, x, p, pbar, 0);
      expect(rc == 0 && isfinite(o[nrows * H * d - 1]), "causal forward rows");
    }
  /* outputs other than o may be absent */
  expect(oracle_forward_rows(q, rb, rp, nrows, k, v, L, L, B, H, Hkv, d, bs, 1.5, 4.0, 1.0, 1, 1,
                             summ, nb, 0, o, NULL, NULL, NULL, NULL, 1) == 0,
         "forward rows without optional outputs");
  /* non-causal: every complete block of n_kv keys is a candidate */
  expect(oracle_forward_rows(q, rb, rp, 4, k, v, L, L, B, H, Hkv, d, bs, 1.5, 4.0, 1.0, 1, 0,
                             summ, nb, nb, o, tau, x, p, pbar, 1) == 0,
         "non-causal forward rows");
  /* argument checks */
  expect(oracle_forward_rows(q, rb, rp, 1, k, v, L, L, B, 3, Hkv, d, bs, 1.5, 4.0, 1.0, 1, 1,
                             summ, nb, 0, o, NULL, NULL, NULL, NULL, 1) == -1, "H % Hkv rejected");
  expect(oracle_forward_rows(q, rb, rp, 1, k, v, L, L, B, H, Hkv, d, bs, 2.5, 4.0, 1.0, 1, 1,
                             summ, nb, 0, o, NULL, NULL, NULL, NULL, 1) == -1, "alpha rejected");
  expect(oracle_forward_rows(q, rb, rp, 1, k, v, L, L, B, H, Hkv, d, bs, 1.5, 4.0, -1.0, 1, 1,
                             summ, nb, 0, o, NULL, NULL, NULL, NULL, 1) == -1, "sigma rejected");
  expect(oracle_forward_rows(q, rb, rp, 1, k, v, L, 100, B, H, Hkv, d, bs, 1.5, 4.0, 1.0, 1, 0,
                             summ, nb, 0, o, NULL, NULL, NULL, NULL, 1) == -1,
         "ragged non-causal keys rejected");
  free(k); free(v); free(w); free(summ); free(q); free(rb); free(rp);
  free(o); free(tau); free(x); free(p); free(pbar);
}

static void run_backward(void) {
  const int B = 1, H = 4, Hkv = 2, N = 192, d = 16, bs = 64;
  float* q = randf((size_t)B * H * N * d, 2.0);
  float* k = randf((size_t)B * Hkv * N * d, 1.0);
  float* v = randf((size_t)B * Hkv * N * d, 1.0);
  float* w = randf((size_t)d * d, 0.3);
  float* dout = randf((size_t)B * H * N * d, 1.0);
  double* dq = (double*)malloc(sizeof(double) * B * H * N * d);
  double* dk = (double*)malloc(sizeof(double) * B * Hkv * N * d);
  double* dv = (double*)malloc(sizeof(double) * B * Hkv * N * d);
  double* dws = (double*)malloc(sizeof(double) * d * d);
  const double alphas[] = {1.25, 1.5, 2.0};
  for (int ai = 0; ai < 3; ++ai)
    for (int window = 1; window <= 2; ++window) {
      const int rc = oracle_prefill_backward(q, k, v, w, dout, B, H, Hkv, N, d, bs, alphas[ai],
                                             4.0, window == 2 ? 0.5 : 1.0, window, dq, dk, dv,
                                             dws, 0);
      expect(rc == 0 && isfinite(dws[d * d - 1]) && isfinite(dq[0]), "prefill backward");
    }
  expect(oracle_prefill_backward(q, k, v, w, dout, B, 3, Hkv, N, d, bs, 1.5, 4.0, 1.0, 1, dq, dk,
                                 dv, dws, 1) == -1, "backward H % Hkv rejected");
  expect(oracle_prefill_backward(q, k, v, w, dout, B, H, Hkv, N, d, bs, 1.0, 4.0, 1.0, 1, dq, dk,
                                 dv, dws, 1) == -1, "backward alpha rejected");
  expect(oracle_prefill_backward(q, k, v, w, dout, B, H, Hkv, N, d, bs, 1.5, 4.0, 1.0, 0, dq, dk,
                                 dv, dws, 1) == -1, "backward window rejected");
  free(q); free(k); free(v); free(w); free(dout); free(dq); free(dk); free(dv); free(dws);
}

int main(void) {
  expect(oracle_max_threads() >= 1, "thread count");
  run_entmax();
  run_summaries();
  run_forward();
  run_backward();
  if (failures) return 1;
  printf("oracle driver: ok\n");
  return 0;
}
