/*
 * dash_oracle.c -- plain, slow CPU reference of the DashAttention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library shares
 * no code, header, table or helper with it.
 *
 * Source: "DashAttention: Differentiable and Adaptive Sparse Hierarchical
 * Attention" explainer pages (gist.science, arXiv 2605.18753; Japanese, Hindi
 * and Arabic copies), section "Technical summary", subsections
 *   Stage 0 - local chunk summarization,
 *   Stage 1 - entmax chunk routing (w = alpha-entmax(gamma * zbar)),
 *   Stage 2 - prior-induced sparse softmax,
 * and the zingnex.cn forum article on DashAttention, section
 * "Technical implementation details / alpha-entmax transform".
 *
 * Every quantity is computed in IEEE double.  Inputs arrive as float32 arrays
 * (bf16 inputs are passed as their exact float32 values) and are promoted
 * element by element.  No blocking, fusion or reordering beyond the stated
 * algorithm: a reader can check each function against the pages by eye.
 *
 * Readings of the pages that this file fixes (the pages leave them open):
 *   R1  coarse score zbar_j = q . s_j / sqrt(d); entmax input x = (alpha-1)*gamma*zbar.
 *   R2  alpha-entmax is the Tsallis entmax: p_j = [x_j - tau]_+^(1/(alpha-1)),
 *       tau the unique root of sum_j p_j = 1.
 *   R3  summary s_j = mean of the block's keys times W_s (the zero-initialised
 *       learned query of Stage 0 pools uniformly); one W_s for all heads, row
 *       vector convention s = m . W_s, W_s row-major [d_in][d_out].
 *   R4  causal: routing candidates are the complete blocks strictly before the
 *       query's own block; the own block is always attended, token-causally,
 *       with zero bias.
 *   R5  GQA: query heads sharing a KV head average their entmax probabilities
 *       (after entmax); every head of the group uses the average pbar.
 *   R6  prior-induced softmax: logit q.k/sqrt(d) + log pbar(block) on routed
 *       blocks (pbar > 0); blocks with pbar = 0 are masked.
 *   R8  prior strength sigma >= 0: the routed-block bias is sigma * log pbar,
 *       i.e. the reference distribution is g proportional to pbar^sigma on the
 *       support (sigma = 1: the routing distribution; sigma = 0: uniform over
 *       the support, the routing then acts as a mask only).
 *   R9  near-diagonal window W >= 1: the query's own block and the W - 1 blocks
 *       before it form the separate branch (bias 0, token-causal, never routed);
 *       routing candidates are the complete blocks j < own - (W - 1).
 *   R3b with a summary query qbar (one d-vector per KV head), the block is
 *       pooled by scaled dot-product attention of qbar over the block's keys,
 *       the keys serving as values: m = sum_t softmax_t(qbar . k_t / sqrt(d)) k_t,
 *       then s_j = m . W_s as in R3.  qbar = 0 gives R3's uniform mean.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* alpha-entmax (Stage 1).                                                  */
/* ------------------------------------------------------------------------ */

static int cmp_desc(const void* a, const void* b) {
  double x = *(const double*)a, y = *(const double*)b;
  return (x < y) - (x > y);
}

/* alpha = 2 (sparsemax, the case the forum article credits to Martins &
 * Astudillo 2016): sort descending; the support size k* is the largest k with
 * 1 + k x_(k) > sum_{r<=k} x_(r); tau = (sum_{r<=k*} x_(r) - 1) / k*. */
static double tau_sparsemax(const double* xs_desc, int n) {
  double csum = 0.0, tau = 0.0;
  for (int k = 1; k <= n; ++k) {
    csum += xs_desc[k - 1];
    if (1.0 + k * xs_desc[k - 1] > csum) tau = (csum - 1.0) / k;
  }
  return tau;
}

/* alpha = 1.5, exact by sorting (Peters, Niculae & Martins 2019): for the
 * top-k set, tau_k solves sum_{r<=k} (x_(r) - tau)^2 = 1 on the branch
 * tau < mean, i.e. tau_k = M_k - sqrt(1/k - (S_k - M_k^2)) with M_k the mean
 * and S_k the mean square of the top k.  k* is the largest k whose root is
 * real and lies strictly below x_(k). */
static double tau_entmax15(const double* xs_desc, int n) {
  double s1 = 0.0, s2 = 0.0, tau = xs_desc[0] - 1.0;
  for (int k = 1; k <= n; ++k) {
    double xk = xs_desc[k - 1];
    s1 += xk;
    s2 += xk * xk;
    double m = s1 / k, msq = s2 / k;
    double rad = 1.0 / k - (msq - m * m);
    if (rad < 0.0) continue;
    double tk = m - sqrt(rad);
    if (tk < xk) tau = tk;
  }
  return tau;
}

/* any alpha in (1, 2]: bisection of f(tau) = sum_j [x_j - tau]_+^(1/(alpha-1)) - 1
 * on the bracket [x_max - 1, x_max - n^(1-alpha)] where f changes sign. */
static double tau_bisect(const double* x, int n, double alpha) {
  double xmax = x[0];
  for (int j = 1; j < n; ++j) xmax = x[j] > xmax ? x[j] : xmax;
  double e = 1.0 / (alpha - 1.0);
  double lo = xmax - 1.0, hi = xmax - pow((double)n, 1.0 - alpha);
  for (int it = 0; it < 200; ++it) {
    double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    double f = -1.0;
    for (int j = 0; j < n; ++j)
      if (x[j] > mid) f += pow(x[j] - mid, e);
    if (f > 0.0) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

/* p = alpha-entmax over n inputs already in threshold units x = (alpha-1)*y.
 * method: 0 = automatic (sort for alpha 2 and 1.5, bisection otherwise),
 *         1 = always bisection.  Returns tau.  Bisection results are
 *         renormalised by their sum; the sort-based roots are exact. */
double oracle_entmax(const double* x, int n, double alpha, int method, double* p) {
  if (n <= 0) return NAN;
  double tau;
  int use_sort = method == 0 && (alpha == 2.0 || alpha == 1.5);
  if (use_sort) {
    double* xs = (double*)malloc(sizeof(double) * n);
    memcpy(xs, x, sizeof(double) * n);
    qsort(xs, n, sizeof(double), cmp_desc);
    tau = alpha == 2.0 ? tau_sparsemax(xs, n) : tau_entmax15(xs, n);
    free(xs);
  } else {
    tau = tau_bisect(x, n, alpha);
  }
  double e = 1.0 / (alpha - 1.0), sum = 0.0;
  for (int j = 0; j < n; ++j) {
    p[j] = x[j] > tau ? pow(x[j] - tau, e) : 0.0;
    sum += p[j];
  }
  if (!use_sort && sum > 0.0)
    for (int j = 0; j < n; ++j) p[j] /= sum;
  return tau;
}

/* ------------------------------------------------------------------------ */
/* Stage 0: block summaries.                                                */
/* ------------------------------------------------------------------------ */

/* k: [B, Hkv, kv_stride, d] float32; blocks [0, nblocks) must be complete.
 * q_bar: NULL (uniform pooling, R3) or [Hkv, d] float32 summary queries (R3b).
 * out: [B, Hkv, nblocks, d] double.
 *   weights  e_t = 1                                           (q_bar NULL)
 *            e_t = exp(z_t - max_u z_u), z_t = qbar_h . k_t / sqrt(d)
 *   pooled   m = sum_{t in j} e_t k_t / sum_{t in j} e_t
 *   summary  s_j = m . W_s */
void oracle_summaries(const float* k, int B, int Hkv, int64_t kv_stride, int d, int bs,
                      int64_t nblocks, const float* w_s, const float* q_bar, double* out) {
  int64_t units = (int64_t)B * Hkv * nblocks;
#pragma omp parallel for schedule(static)
  for (int64_t u = 0; u < units; ++u) {
    int64_t j = u % nblocks, bh = u / nblocks;
    int h = (int)(bh % Hkv);
    const float* kb = k + (bh * kv_stride + j * bs) * d;
    double* e = (double*)malloc(sizeof(double) * bs);
    double esum = 0.0;
    if (q_bar == NULL) {
      for (int t = 0; t < bs; ++t) e[t] = 1.0;
    } else {
      const float* qb = q_bar + (int64_t)h * d;
      double zmax = -INFINITY;
      for (int t = 0; t < bs; ++t) {
        double z = 0.0;
        for (int c = 0; c < d; ++c) z += (double)qb[c] * (double)kb[(int64_t)t * d + c];
        e[t] = z / sqrt((double)d);
        if (e[t] > zmax) zmax = e[t];
      }
      for (int t = 0; t < bs; ++t) e[t] = exp(e[t] - zmax);
    }
    for (int t = 0; t < bs; ++t) esum += e[t];
    double* m = (double*)calloc(d, sizeof(double));
    for (int t = 0; t < bs; ++t)
      for (int c = 0; c < d; ++c) m[c] += e[t] * (double)kb[(int64_t)t * d + c];
    for (int c = 0; c < d; ++c) m[c] /= esum;
    double* s = out + u * d;
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int r = 0; r < d; ++r) acc += m[r] * (double)w_s[(int64_t)r * d + c];
      s[c] = acc;
    }
    free(m);
    free(e);
  }
}

/* ------------------------------------------------------------------------ */
/* Stages 1 and 2 for a list of query rows.                                 */
/* ------------------------------------------------------------------------ */

/*
 * One query row = one (sequence b, query position i) with all H heads.
 *   q_rows : [nrows, H, d] float32, the row's query vectors
 *   row_b, row_pos : [nrows] sequence index and position of each row
 *   k, v   : [B, Hkv, kv_stride, d] float32
 *   n_kv   : valid keys per sequence (non-causal only; causal uses i + 1)
 *   summ   : [B, Hkv, summ_stride, d] double, summaries of complete blocks
 *   causal : 1 = rules R4 and R9; 0 = every block of the n_kv keys is a
 *            candidate (n_kv % bs == 0 required) and there is no own block.
 *   sigma  : prior strength (R8), >= 0
 *   window : near-diagonal window in blocks (R9), >= 1
 * Outputs (each may be NULL except o):
 *   o      : [nrows, H, d]
 *   tau    : [nrows, H]                 NaN when the row has no candidate
 *   x_out  : [nrows, H, nb_out]         entmax inputs, NaN off the candidates
 *   p_out  : [nrows, H, nb_out]         per-head entmax probabilities
 *   pbar   : [nrows, Hkv, nb_out]       group-averaged probabilities
 * Returns 0, or -1 on invalid arguments.
 */
int oracle_forward_rows(const float* q_rows, const int64_t* row_b, const int64_t* row_pos,
                        int64_t nrows, const float* k, const float* v, int64_t kv_stride,
                        int64_t n_kv, int B, int H, int Hkv, int d, int bs, double alpha,
                        double gamma, double sigma, int window, int causal, const double* summ,
                        int64_t summ_stride, int64_t nb_out, double* o, double* tau,
                        double* x_out, double* p_out, double* pbar, int nthreads) {
  if (H % Hkv != 0 || alpha <= 1.0 || alpha > 2.0 || bs <= 0 || d <= 0) return -1;
  if (!(sigma >= 0.0) || window < 1) return -1;
  if (!causal && n_kv % bs != 0) return -1;
  const int G = H / Hkv;
  const double inv_sqrt_d = 1.0 / sqrt((double)d);
  int err = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t b = row_b[r], i = row_pos[r];
    if (b < 0 || b >= B || i < 0 || i >= kv_stride) {
#pragma omp atomic write
      err = 1;
      continue;
    }
    const int64_t own = i / bs;
    /* first block of the near-diagonal branch; candidates are the blocks before it */
    const int64_t win0 = own - (window - 1) > 0 ? own - (window - 1) : 0;
    const int64_t ncand = causal ? win0 : n_kv / bs;
    if (ncand > summ_stride || (nb_out > 0 && ncand > nb_out)) {
#pragma omp atomic write
      err = 1;
      continue;
    }

    double* x = (double*)malloc(sizeof(double) * (ncand > 0 ? ncand : 1) * H);
    double* p = (double*)malloc(sizeof(double) * (ncand > 0 ? ncand : 1) * H);
    double* pb = (double*)calloc((ncand > 0 ? ncand : 1) * Hkv, sizeof(double));

    /* Stage 1: coarse scores against the summaries, entmax per head. */
    for (int h = 0; h < H; ++h) {
      const int g = h / G;
      const float* qv = q_rows + (r * H + h) * (int64_t)d;
      for (int64_t j = 0; j < ncand; ++j) {
        const double* s = summ + (((int64_t)b * Hkv + g) * summ_stride + j) * d;
        double z = 0.0;
        for (int c = 0; c < d; ++c) z += (double)qv[c] * s[c];
        x[h * ncand + j] = (alpha - 1.0) * gamma * z * inv_sqrt_d;
      }
      double t = ncand > 0 ? oracle_entmax(x + h * ncand, (int)ncand, alpha, 0, p + h * ncand)
                           : NAN;
      if (tau) tau[r * H + h] = t;
    }
    /* GQA: average the probabilities of the heads that share a KV head. */
    for (int h = 0; h < H; ++h)
      for (int64_t j = 0; j < ncand; ++j) pb[(h / G) * ncand + j] += p[h * ncand + j] / G;

    if (x_out || p_out || pbar) {
      for (int h = 0; h < H; ++h)
        for (int64_t j = 0; j < nb_out; ++j) {
          if (x_out) x_out[(r * H + h) * nb_out + j] = j < ncand ? x[h * ncand + j] : NAN;
          if (p_out) p_out[(r * H + h) * nb_out + j] = j < ncand ? p[h * ncand + j] : 0.0;
        }
      if (pbar)
        for (int g = 0; g < Hkv; ++g)
          for (int64_t j = 0; j < nb_out; ++j)
            pbar[((int64_t)r * Hkv + g) * nb_out + j] = j < ncand ? pb[g * ncand + j] : 0.0;
    }

    /* Stage 2: softmax over the keys of routed blocks (bias sigma log pbar)
     * and the near-diagonal branch: keys win0 * bs .. i (bias 0). */
    const int64_t nkeys_max = (ncand + (causal ? window : 0)) * (int64_t)bs;
    double* logit = (double*)malloc(sizeof(double) * nkeys_max);
    int64_t* key = (int64_t*)malloc(sizeof(int64_t) * nkeys_max);
    for (int h = 0; h < H; ++h) {
      const int g = h / G;
      const float* qv = q_rows + (r * H + h) * (int64_t)d;
      const float* kg = k + ((int64_t)b * Hkv + g) * kv_stride * d;
      const float* vg = v + ((int64_t)b * Hkv + g) * kv_stride * d;
      int64_t nk = 0;
      for (int64_t j = 0; j < ncand; ++j) {
        double pj = pb[g * ncand + j];
        if (!(pj > 0.0)) continue;
        for (int64_t t = j * bs; t < (j + 1) * bs; ++t) {
          key[nk] = t;
          logit[nk++] = sigma * log(pj);
        }
      }
      if (causal)
        for (int64_t t = win0 * bs; t <= i; ++t) {
          key[nk] = t;
          logit[nk++] = 0.0;
        }
      double mx = -INFINITY;
      for (int64_t a = 0; a < nk; ++a) {
        const float* kt = kg + key[a] * d;
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += (double)qv[c] * (double)kt[c];
        logit[a] += dot * inv_sqrt_d;
        if (logit[a] > mx) mx = logit[a];
      }
      double* ov = o + (r * H + h) * (int64_t)d;
      for (int c = 0; c < d; ++c) ov[c] = 0.0;
      double den = 0.0;
      for (int64_t a = 0; a < nk; ++a) {
        double w = exp(logit[a] - mx);
        den += w;
        const float* vt = vg + key[a] * d;
        for (int c = 0; c < d; ++c) ov[c] += w * (double)vt[c];
      }
      for (int c = 0; c < d; ++c) ov[c] = nk > 0 ? ov[c] / den : NAN;
    }
    free(logit);
    free(key);
    free(x);
    free(p);
    free(pb);
  }
  return err ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Backward of the causal prefill (mean-pooled summaries, rule R3).         */
/* ------------------------------------------------------------------------ */

/*
 * The pages (explainer, "Technical summary" and "Contributions") stress that
 * the hierarchy is differentiable end to end: alpha-entmax carries gradients
 * from the fine attention back through the routing into the summaries.  This
 * is the chain rule of oracle_forward_rows (causal, R1-R9) for one scalar
 * loss L = sum(o * dO), one query row at a time, in IEEE double:
 *   Stage 2   P = softmax(l), l_t = q.k_t/sqrt(d) + bias_t, o = sum_t P_t v_t
 *             dv_t += P_t dO;  dl_t = P_t (dO.v_t - dO.o)
 *             dq += sum_t dl_t k_t / sqrt(d);  dk_t += dl_t q / sqrt(d)
 *             bias of a routed block j is sigma log pbar_j:
 *             dpbar_j = sigma (sum_{t in j} dl_t) / pbar_j
 *   GQA       pbar_j = (1/G) sum_h p_{h,j}:  dp_{h,j} = dpbar_j / G
 *   Stage 1   p = alpha-entmax(x); on the support dp/dx = (diag(u) - u u^T /
 *             sum u) / (alpha - 1) with u = p^(2-alpha), zero elsewhere;
 *             x = (alpha-1) gamma q.s_j/sqrt(d), so
 *             dzbar_j = gamma (u_j dp_j - u_j (u.dp) / sum u)
 *             dq += sum_j dzbar_j s_j / sqrt(d);  ds_j += dzbar_j q / sqrt(d)
 *   Stage 0   s_j = m_j W_s with m_j the mean of block j's keys:
 *             dW_s += m_j^T ds_j;  dk_t += (ds_j W_s^T) / bs for t in block j
 * Blocks with pbar = 0 are masked and take no gradient.
 *   q, d_o [B, H, N, d]; k, v [B, Hkv, N, d]; w_s [d, d] (float32 values)
 *   dq [B, H, N, d]; dk, dv [B, Hkv, N, d]; dws [d, d] (double, overwritten)
 * The (sequence, KV head) pairs run in parallel: each owns its rows of dq,
 * dk, dv and ds, so no output is written by two threads.  Returns 0, or -1
 * on invalid arguments.
 */
int oracle_prefill_backward(const float* q, const float* k, const float* v, const float* w_s,
                            const float* d_o, int B, int H, int Hkv, int64_t N, int d, int bs,
                            double alpha, double gamma, double sigma, int window, double* dq,
                            double* dk, double* dv, double* dws, int nthreads) {
  if (B < 1 || H < 1 || Hkv < 1 || H % Hkv != 0 || N < 1 || d < 1 || bs < 1) return -1;
  if (alpha <= 1.0 || alpha > 2.0 || !(sigma >= 0.0) || window < 1) return -1;
  const int G = H / Hkv;
  const int64_t nb = N / bs;                     /* complete blocks */
  const double rs = 1.0 / sqrt((double)d);
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const int64_t nbg = (int64_t)B * Hkv;
  /* block means m and summaries s = m W_s, per (b, g) */
  double* m = (double*)calloc((size_t)(nbg * (nb > 0 ? nb : 1) * d), sizeof(double));
  double* s = (double*)calloc((size_t)(nbg * (nb > 0 ? nb : 1) * d), sizeof(double));
  double* ds = (double*)calloc((size_t)(nbg * (nb > 0 ? nb : 1) * d), sizeof(double));
  memset(dq, 0, sizeof(double) * (size_t)(B * (int64_t)H * N * d));
  memset(dk, 0, sizeof(double) * (size_t)(nbg * N * d));
  memset(dv, 0, sizeof(double) * (size_t)(nbg * N * d));
  for (int64_t u = 0; u < nbg * nb; ++u) {
    const int64_t bg = u / nb, j = u % nb;
    const float* kb = k + (bg * N + j * bs) * d;
    double* mj = m + u * d;
    for (int t = 0; t < bs; ++t)
      for (int c = 0; c < d; ++c) mj[c] += (double)kb[(int64_t)t * d + c];
    for (int c = 0; c < d; ++c) mj[c] /= bs;
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int r = 0; r < d; ++r) acc += mj[r] * (double)w_s[(int64_t)r * d + c];
      s[u * d + c] = acc;
    }
  }

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bg = 0; bg < nbg; ++bg) {
    const int64_t b = bg / Hkv;
    const int g = (int)(bg % Hkv);
    const int64_t nc_max = nb > 0 ? nb : 1;
    double* x = (double*)malloc(sizeof(double) * nc_max);
    double* p = (double*)malloc(sizeof(double) * nc_max * G);
    double* pbar = (double*)malloc(sizeof(double) * nc_max);
    double* dlogpbar = (double*)malloc(sizeof(double) * nc_max);
    double* dpbar = (double*)malloc(sizeof(double) * nc_max);
    const int64_t nkeys_max = (nb + window + 1) * (int64_t)bs;
    int64_t* key = (int64_t*)malloc(sizeof(int64_t) * nkeys_max);
    double* logit = (double*)malloc(sizeof(double) * nkeys_max);
    double* P = (double*)malloc(sizeof(double) * nkeys_max);
    double* orow = (double*)malloc(sizeof(double) * d);
    const float* kg = k + bg * N * d;
    const float* vg = v + bg * N * d;
    double* dkg = dk + bg * N * d;
    double* dvg = dv + bg * N * d;
    for (int64_t i = 0; i < N; ++i) {
      const int64_t own = i / bs;
      const int64_t win0 = own - (window - 1) > 0 ? own - (window - 1) : 0;
      const int64_t ncand = win0 < nb ? win0 : nb;
      /* Stage 1 forward: entmax per head, then the group average */
      for (int64_t j = 0; j < ncand; ++j) pbar[j] = 0.0;
      for (int hh = 0; hh < G; ++hh) {
        const float* qv = q + (((b * H) + g * G + hh) * N + i) * d;
        for (int64_t j = 0; j < ncand; ++j) {
          const double* sj = s + (bg * nb + j) * d;
          double z = 0.0;
          for (int c = 0; c < d; ++c) z += (double)qv[c] * sj[c];
          x[j] = (alpha - 1.0) * gamma * z * rs;
        }
        if (ncand > 0) oracle_entmax(x, (int)ncand, alpha, 0, p + hh * ncand);
        for (int64_t j = 0; j < ncand; ++j) pbar[j] += p[hh * ncand + j] / G;
      }
      /* Stage 2 keys: routed blocks (bias sigma log pbar), then the branch */
      int64_t nk = 0, nrt = 0;
      for (int64_t j = 0; j < ncand; ++j) {
        if (!(pbar[j] > 0.0)) continue;
        for (int64_t t = j * bs; t < (j + 1) * bs; ++t) {
          key[nk] = t;
          logit[nk++] = sigma * log(pbar[j]);
        }
      }
      nrt = nk;
      for (int64_t t = win0 * bs; t <= i; ++t) {
        key[nk] = t;
        logit[nk++] = 0.0;
      }
      for (int64_t j = 0; j < ncand; ++j) dlogpbar[j] = 0.0;
      for (int hh = 0; hh < G; ++hh) {
        const int64_t hrow = ((b * H) + g * G + hh) * N + i;
        const float* qv = q + hrow * d;
        const float* dov = d_o + hrow * d;
        double* dqv = dq + hrow * d;
        double mx = -INFINITY;
        for (int64_t a = 0; a < nk; ++a) {
          const float* kt = kg + key[a] * d;
          double dot = 0.0;
          for (int c = 0; c < d; ++c) dot += (double)qv[c] * (double)kt[c];
          P[a] = logit[a] + dot * rs;
          if (P[a] > mx) mx = P[a];
        }
        double den = 0.0;
        for (int64_t a = 0; a < nk; ++a) {
          P[a] = exp(P[a] - mx);
          den += P[a];
        }
        for (int c = 0; c < d; ++c) orow[c] = 0.0;
        for (int64_t a = 0; a < nk; ++a) {
          P[a] /= den;
          const float* vt = vg + key[a] * d;
          for (int c = 0; c < d; ++c) orow[c] += P[a] * (double)vt[c];
        }
        double doo = 0.0;
        for (int c = 0; c < d; ++c) doo += (double)dov[c] * orow[c];
        for (int64_t a = 0; a < nk; ++a) {
          const float* kt = kg + key[a] * d;
          const float* vt = vg + key[a] * d;
          double dov_v = 0.0;
          for (int c = 0; c < d; ++c) dov_v += (double)dov[c] * (double)vt[c];
          const double dl = P[a] * (dov_v - doo);
          double* dkt = dkg + key[a] * d;
          double* dvt = dvg + key[a] * d;
          for (int c = 0; c < d; ++c) {
            dvt[c] += P[a] * (double)dov[c];
            dqv[c] += dl * (double)kt[c] * rs;
            dkt[c] += dl * (double)qv[c] * rs;
          }
          if (a < nrt) dlogpbar[key[a] / bs] += sigma * dl;
        }
      }
      if (ncand == 0) continue;
      /* through the bias into pbar, the group average and each head's entmax */
      for (int64_t j = 0; j < ncand; ++j) dpbar[j] = pbar[j] > 0.0 ? dlogpbar[j] / pbar[j] : 0.0;
      for (int hh = 0; hh < G; ++hh) {
        const int64_t hrow = ((b * H) + g * G + hh) * N + i;
        const float* qv = q + hrow * d;
        double* dqv = dq + hrow * d;
        const double* ph = p + hh * ncand;
        double su = 0.0, sud = 0.0;
        for (int64_t j = 0; j < ncand; ++j) {
          const double u = ph[j] > 0.0 ? pow(ph[j], 2.0 - alpha) : 0.0;
          su += u;
          sud += u * dpbar[j] / G;
        }
        for (int64_t j = 0; j < ncand; ++j) {
          const double u = ph[j] > 0.0 ? pow(ph[j], 2.0 - alpha) : 0.0;
          const double dz = gamma * (u * dpbar[j] / G - u * sud / su);
          if (dz == 0.0) continue;
          const double* sj = s + (bg * nb + j) * d;
          double* dsj = ds + (bg * nb + j) * d;
          for (int c = 0; c < d; ++c) {
            dqv[c] += dz * sj[c] * rs;
            dsj[c] += dz * (double)qv[c] * rs;
          }
        }
      }
    }
    /* Stage 0: the block means carry ds_j W_s^T / bs to every key of block j */
    for (int64_t j = 0; j < nb; ++j) {
      const double* dsj = ds + (bg * nb + j) * d;
      for (int r = 0; r < d; ++r) {
        double dm = 0.0;
        for (int c = 0; c < d; ++c) dm += dsj[c] * (double)w_s[(int64_t)r * d + c];
        for (int64_t t = j * bs; t < (j + 1) * bs; ++t) dkg[t * d + r] += dm / bs;
      }
    }
    free(x);
    free(p);
    free(pbar);
    free(dlogpbar);
    free(dpbar);
    free(key);
    free(logit);
    free(P);
    free(orow);
  }
  /* dW_s = sum over every (b, g, j) of m_j^T ds_j */
  for (int r = 0; r < d; ++r)
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t u = 0; u < nbg * nb; ++u) acc += m[u * d + r] * ds[u * d + c];
      dws[(int64_t)r * d + c] = acc;
    }
  free(m);
  free(s);
  free(ds);
  return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
