/*
 * Host-side driver for running the C oracle (oracle/gdr_oracle.c, test
 * infrastructure) under AddressSanitizer and UndefinedBehaviorSanitizer.
 * It calls every entry point on small deterministic inputs that cover the
 * edge cases the tests use (an empty sequence, a one-token sequence, a
 * packed batch, grouped heads, NULL optional outputs, pair lists, the erase
 * term off) and prints one checksum per call, so that a sanitized and a
 * plain build can be compared.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int gdr_oracle_gates(int64_t total, int H_k, int H_v, int d_k, double scale, double l2_eps,
                     const double *q, const double *k, const double *a, const double *b,
                     const double *A_log, const double *dt_bias, double *q_hat, double *k_hat,
                     double *g, double *beta);
int gdr_oracle_fwd(int64_t num_seqs, const int64_t *cu_seqlens, int H_k, int H_v, int d_k, int d_v,
                   double scale, double l2_eps, int erase, const double *q, const double *k,
                   const double *v, const double *a, const double *b, const double *A_log,
                   const double *dt_bias, const double *init_state, double *o,
                   double *final_state, const int64_t *pairs, int64_t n_pairs, int n_threads);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double next_uniform(void) {  /* xorshift64*, in [-1, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 0x2545f4914f6cdd1dull) >> 11) / 4503599627370496.0 - 1.0;
}
static double *fill(size_t n) {
  double *x = malloc(sizeof(double) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) x[i] = next_uniform();
  return x;
}
static double sum(const double *x, size_t n) {
  double s = 0.0;
  for (size_t i = 0; i < n; ++i) s += x[i] * (double)((i % 7) + 1);
  return s;
}

int main(void) {
  const int H_k = 2, H_v = 4, d_k = 16, d_v = 8;
  const int64_t cu[] = {0, 0, 1, 19, 52};  /* empty, one token, two longer */
  const int64_t N = 4, T = cu[4];
  double *q = fill((size_t)T * H_k * d_k), *k = fill((size_t)T * H_k * d_k);
  double *v = fill((size_t)T * H_v * d_v), *a = fill((size_t)T * H_v), *b = fill((size_t)T * H_v);
  double *A_log = fill(H_v), *dt_bias = fill(H_v);
  double *s0 = fill((size_t)N * H_v * d_k * d_v);
  double *o = calloc((size_t)T * H_v * d_v, sizeof(double));
  double *sT = calloc((size_t)N * H_v * d_k * d_v, sizeof(double));
  double *qh = calloc((size_t)T * H_k * d_k, sizeof(double)), *kh = calloc((size_t)T * H_k * d_k, sizeof(double));
  double *g = calloc((size_t)T * H_v, sizeof(double)), *beta = calloc((size_t)T * H_v, sizeof(double));
  const size_t no = (size_t)T * H_v * d_v, ns = (size_t)N * H_v * d_k * d_v;
  int rc = gdr_oracle_gates(T, H_k, H_v, d_k, 0.25, 1e-6, q, k, a, b, A_log, dt_bias, qh, kh, g, beta);
  printf("gates %d %.17g %.17g\n", rc, sum(qh, (size_t)T * H_k * d_k), sum(g, (size_t)T * H_v));
  rc = gdr_oracle_gates(T, H_k, H_v, d_k, 0.25, 1e-6, q, k, a, b, A_log, dt_bias, NULL, kh, NULL, beta);
  printf("gates-partial %d %.17g\n", rc, sum(beta, (size_t)T * H_v));
  rc = gdr_oracle_fwd(N, cu, H_k, H_v, d_k, d_v, 0.25, 1e-6, 1, q, k, v, a, b, A_log, dt_bias, s0,
                      o, sT, NULL, 0, 1);
  printf("fwd %d %.17g %.17g\n", rc, sum(o, no), sum(sT, ns));
  rc = gdr_oracle_fwd(N, cu, H_k, H_v, d_k, d_v, 0.25, 1e-6, 1, q, k, v, a, b, A_log, dt_bias, NULL,
                      o, NULL, NULL, 0, 1);
  printf("fwd-zero-state %d %.17g\n", rc, sum(o, no));
  rc = gdr_oracle_fwd(N, cu, H_k, H_v, d_k, d_v, 0.25, 1e-6, 0, q, k, v, a, b, A_log, dt_bias, s0,
                      NULL, sT, NULL, 0, 1);
  printf("fwd-no-erase %d %.17g\n", rc, sum(sT, ns));
  const int64_t pairs[] = {3, 1, 1, 3, 0, 0};
  rc = gdr_oracle_fwd(N, cu, H_k, H_v, d_k, d_v, 0.25, 1e-6, 1, q, k, v, a, b, A_log, dt_bias, s0,
                      o, sT, pairs, 3, 1);
  printf("fwd-pairs %d %.17g %.17g\n", rc, sum(o, no), sum(sT, ns));
  const int64_t bad[] = {9, 0};
  rc = gdr_oracle_fwd(N, cu, H_k, H_v, d_k, d_v, 0.25, 1e-6, 1, q, k, v, a, b, A_log, dt_bias, s0,
                      o, sT, bad, 1, 1);
  printf("fwd-bad-pair %d\n", rc);
  rc = gdr_oracle_fwd(N, cu, 3, H_v, d_k, d_v, 0.25, 1e-6, 1, q, k, v, a, b, A_log, dt_bias, s0, o,
                      sT, NULL, 0, 1);
  printf("fwd-bad-shape %d\n", rc);
  free(q); free(k); free(v); free(a); free(b); free(A_log); free(dt_bias); free(s0); free(o);
  free(sT); free(qh); free(kh); free(g); free(beta);
  return 0;
}
