/*
 * gdr_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The plain, slow, fp64 CPU definition of the gated delta rule, used by the
 * tests, by the smoke check and by the CPU-baseline leg of the benchmark to
 * check the GPU library.  Nothing in the product path may link, load or call
 * this file; it shares no code, header or table with the GPU library.
 *
 * What it computes (one sequential pass per (sequence, value head), exactly in
 * the order the definition states it):
 *
 *   GatedDeltaRule.ixx File Reference, "Detailed Description":
 *     per value head a state S of shape [d_k, d_v]; each step
 *       S     <- S * exp(g_t)
 *       delta <- (v_t - k_t^T S) * beta_t
 *       S     <- S + k_t (outer) delta
 *       o_t   <- q_t^T S
 *     with q and k L2-normalized and q scaled by 1/sqrt(d_k); the gates are
 *     derived inside from the raw projections a, b and the per-head
 *     parameters A_log, dt_bias:
 *       beta = sigmoid(b),   g = -exp(A_log) * softplus(a + dt_bias).
 *
 *   Track L -- genuine gated delta rule + Mamba2 SSM (tessera PR #77),
 *   "The core finding (L0)": with the erase term removed the same recurrence
 *   becomes gated linear attention, S <- alpha*S + beta*k*v^T.  The `erase`
 *   switch below exists only so that the tests can pin that reduction; the
 *   GPU library has no such switch.
 *
 * Readings of points the pages leave open:
 *   - value head h reads key head h / (H_v / H_k) (contiguous groups);
 *   - q has the key heads' layout [tokens, H_k, d_k];
 *   - L2 normalisation is x / sqrt(sum x^2 + l2_eps), l2_eps given by caller;
 *   - softplus(x) = max(x,0) + log1p(exp(-|x|)), with no threshold;
 *   - A_log and dt_bias hold one value per value head.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math), so
 * that every multiply and add is rounded as written.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus as a sum of a ramp and a correction that never overflows. */
static double oracle_softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

static double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Row norm factor 1/sqrt(sum x^2 + eps) of one d-vector. */
static double oracle_inv_norm(const double *x, int d, double eps) {
  double ss = 0.0;
  for (int i = 0; i < d; ++i) ss += x[i] * x[i];
  return 1.0 / sqrt(ss + eps);
}

int gdr_oracle_abi_version(void) { return 1; }

/*
 * Planted-mistake switch, used only by the tests that prove the pins are not
 * vacuous: each nonzero value changes exactly one step of the definition, and
 * every such change must make at least one pin fail.  0 (the default) is the
 * definition itself.
 *   1  drop the erase term            (delta = beta * v)
 *   2  read the output before the write
 *   3  decay after the erase          (delta from the undecayed state)
 *   4  key not normalised
 *   5  1/sqrt(d_k) applied to k instead of q
 *   6  value head h reads key head h % H_k
 *   7  softplus replaced by exp
 *   8  sign of g flipped
 *   9  beta = sigmoid(-b)
 *  10  output read through the transposed state (square states only)
 */
static int oracle_mutation = 0;
void gdr_oracle_set_mutation(int m) { oracle_mutation = m; }
int gdr_oracle_get_mutation(void) { return oracle_mutation; }

/*
 * Gates and normalised q/k, exactly as the component derives them
 * (GatedDeltaRule.ixx File Reference, "Detailed Description").
 *   q, k   : [total, H_k, d_k]        a, b : [total, H_v]
 *   A_log, dt_bias : [H_v]
 *   q_hat, k_hat : [total, H_k, d_k]  (q_hat includes `scale`)
 *   g, beta : [total, H_v]
 * Any output pointer may be NULL (skipped).
 */
int gdr_oracle_gates(int64_t total, int H_k, int H_v, int d_k, double scale, double l2_eps,
                     const double *q, const double *k, const double *a, const double *b,
                     const double *A_log, const double *dt_bias, double *q_hat, double *k_hat,
                     double *g, double *beta) {
  if (total < 0 || H_k <= 0 || H_v <= 0 || d_k <= 0 || H_v % H_k != 0) return 2;
  for (int64_t t = 0; t < total; ++t) {
    for (int hk = 0; hk < H_k; ++hk) {
      const double *qr = q + (t * H_k + hk) * d_k;
      const double *kr = k + (t * H_k + hk) * d_k;
      double iq = oracle_inv_norm(qr, d_k, l2_eps) * scale;
      double ik = oracle_inv_norm(kr, d_k, l2_eps);
      for (int i = 0; i < d_k; ++i) {
        if (q_hat) q_hat[(t * H_k + hk) * d_k + i] = qr[i] * iq;
        if (k_hat) k_hat[(t * H_k + hk) * d_k + i] = kr[i] * ik;
      }
    }
    for (int h = 0; h < H_v; ++h) {
      double x = a[t * H_v + h] + dt_bias[h];
      if (g) g[t * H_v + h] = -exp(A_log[h]) * oracle_softplus(x);
      if (beta) beta[t * H_v + h] = oracle_sigmoid(b[t * H_v + h]);
    }
  }
  return 0;
}

/*
 * The sequential recurrence over one (sequence, value head) pair.
 * S is [d_k, d_v] row-major, updated in place; the token range is [t0, t1).
 */
static void oracle_scan_one(int64_t t0, int64_t t1, int h, int H_k, int H_v, int d_k, int d_v,
                            double scale, double l2_eps, int erase, const double *q,
                            const double *k, const double *v, const double *a, const double *b,
                            const double *A_log, const double *dt_bias, double *S, double *o,
                            double *khat, double *qhat, double *delta) {
  const int m = oracle_mutation;
  const int G = H_v / H_k;
  const int hk = (m == 6) ? h % H_k : h / G;
  for (int64_t t = t0; t < t1; ++t) {
    /* gates: g = -exp(A_log) * softplus(a + dt_bias), alpha = exp(g), beta = sigmoid(b) */
    double x = a[t * H_v + h] + dt_bias[h];
    double sp = (m == 7) ? exp(x) : oracle_softplus(x);
    double gt = -exp(A_log[h]) * sp;
    if (m == 8) gt = -gt;
    double alpha = exp(gt);
    double bt = oracle_sigmoid((m == 9) ? -b[t * H_v + h] : b[t * H_v + h]);
    /* L2-normalised key and query of the shared key head; q also takes `scale` */
    const double *kr = k + (t * H_k + hk) * d_k;
    const double *qr = q + (t * H_k + hk) * d_k;
    double ik = (m == 4) ? 1.0 : oracle_inv_norm(kr, d_k, l2_eps);
    double iq = oracle_inv_norm(qr, d_k, l2_eps);
    if (m == 5)
      ik *= scale;
    else
      iq *= scale;
    for (int i = 0; i < d_k; ++i) {
      khat[i] = kr[i] * ik;
      qhat[i] = qr[i] * iq;
    }
    const double *vr = v + (t * H_v + h) * d_v;
    double *orow = o ? o + (t * H_v + h) * d_v : NULL;
    if (m == 2 && orow) /* planted: read out before the write */
      for (int j = 0; j < d_v; ++j) {
        double acc = 0.0;
        for (int i = 0; i < d_k; ++i) acc += qhat[i] * S[i * d_v + j];
        orow[j] = acc;
      }
    /* S <- S * exp(g)  (planted mistake 3 moves this after the erase read) */
    if (m != 3)
      for (int i = 0; i < d_k * d_v; ++i) S[i] *= alpha;
    /* delta <- (v - k^T S) * beta   (erase off: delta <- v * beta) */
    for (int j = 0; j < d_v; ++j) {
      double u = 0.0;
      if (erase && m != 1)
        for (int i = 0; i < d_k; ++i) u += khat[i] * S[i * d_v + j];
      delta[j] = (vr[j] - u) * bt;
    }
    if (m == 3)
      for (int i = 0; i < d_k * d_v; ++i) S[i] *= alpha;
    /* S <- S + k (outer) delta */
    for (int i = 0; i < d_k; ++i)
      for (int j = 0; j < d_v; ++j) S[i * d_v + j] += khat[i] * delta[j];
    /* o <- q^T S, read after the write */
    if (orow && m != 2) {
      for (int j = 0; j < d_v; ++j) {
        double acc = 0.0;
        for (int i = 0; i < d_k; ++i)
          acc += qhat[i] * ((m == 10 && d_k == d_v) ? S[j * d_v + i] : S[i * d_v + j]);
        orow[j] = acc;
      }
    }
  }
}

/*
 * Full forward pass of the rule.
 *   num_seqs, cu_seqlens[num_seqs+1] (host, int64; cu[0] = 0, nondecreasing)
 *   q, k : [total, H_k, d_k]   v : [total, H_v, d_v]   a, b : [total, H_v]
 *   A_log, dt_bias : [H_v]
 *   init_state : [num_seqs, H_v, d_k, d_v] or NULL (zeros)
 *   o : [total, H_v, d_v] (may be NULL)   final_state : same shape as init (may be NULL)
 *   pairs : optional list of n_pairs (sequence, value head) index pairs; only
 *           those pairs are computed (NULL = all).
 *   erase : 1 = the gated delta rule; 0 = gated linear attention (tests only).
 *   n_threads <= 0 means the OpenMP default.
 * Returns 0, or 2 on a shape error.
 */
int gdr_oracle_fwd(int64_t num_seqs, const int64_t *cu_seqlens, int H_k, int H_v, int d_k, int d_v,
                   double scale, double l2_eps, int erase, const double *q, const double *k,
                   const double *v, const double *a, const double *b, const double *A_log,
                   const double *dt_bias, const double *init_state, double *o,
                   double *final_state, const int64_t *pairs, int64_t n_pairs, int n_threads) {
  if (num_seqs < 0 || H_k <= 0 || H_v <= 0 || d_k <= 0 || d_v <= 0 || H_v % H_k != 0) return 2;
  for (int64_t n = 0; n < num_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return 2;
  const int64_t n_units = pairs ? n_pairs : num_seqs * (int64_t)H_v;
  const size_t sdim = (size_t)d_k * d_v;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#endif
  int err = 0;
#pragma omp parallel
  {
    double *S = (double *)malloc(sizeof(double) * sdim);
    double *khat = (double *)malloc(sizeof(double) * d_k);
    double *qhat = (double *)malloc(sizeof(double) * d_k);
    double *delta = (double *)malloc(sizeof(double) * d_v);
    if (!S || !khat || !qhat || !delta) {
#pragma omp atomic write
      err = 3;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t u = 0; u < n_units; ++u) {
        int64_t n = pairs ? pairs[2 * u] : u / H_v;
        int h = pairs ? (int)pairs[2 * u + 1] : (int)(u % H_v);
        if (n < 0 || n >= num_seqs || h < 0 || h >= H_v) {
#pragma omp atomic write
          err = 2;
          continue;
        }
        size_t soff = ((size_t)n * H_v + h) * sdim;
        if (init_state)
          memcpy(S, init_state + soff, sizeof(double) * sdim);
        else
          memset(S, 0, sizeof(double) * sdim);
        oracle_scan_one(cu_seqlens[n], cu_seqlens[n + 1], h, H_k, H_v, d_k, d_v, scale, l2_eps,
                        erase, q, k, v, a, b, A_log, dt_bias, S, o, khat, qhat, delta);
        if (final_state) memcpy(final_state + soff, S, sizeof(double) * sdim);
      }
    }
    free(S);
    free(khat);
    free(qhat);
    free(delta);
  }
  return err;
}
