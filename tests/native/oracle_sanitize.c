/*
 * oracle_sanitize.c -- drives both CPU oracles (attn_oracle.c,
 * group_norm_oracle.c) under AddressSanitizer and UndefinedBehaviorSanitizer
 * on small cases and on their argument checks.  Test infrastructure: built
 * and run by tests/test_sanitize.py with gcc; exits non-zero on any failed
 * check (a sanitizer report aborts the run by itself).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_attn_f64(const double *q, const double *k, const double *v, double *out, int64_t B,
                    int64_t H, int64_t Lq, int64_t Lk, int64_t d, double scale, int nthreads);
int oracle_attn_rows_f64(const double *q, const double *k, const double *v, int64_t B, int64_t H,
                         int64_t Lq, int64_t Lk, int64_t d, double scale, const int64_t *rows,
                         int64_t nrows, double *out, int nthreads);
int oracle_attn_probs_f64(const double *q, const double *k, const double *v, double *out,
                          double *probs, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                          double scale);
int oracle_group_norm_f64(const double *x, const double *gamma, const double *beta, double *y,
                          int64_t N, int64_t C, int64_t S, int64_t G, double eps, int silu,
                          int nthreads);

static int failures = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static double *rnd(int64_t n, unsigned *state) {
  /* exactly sized heap buffers, so any overrun is reported */
  double *a = malloc((size_t)n * sizeof(double));
  for (int64_t i = 0; i < n; ++i) {
    *state = *state * 1664525u + 1013904223u;
    a[i] = ((double)(*state >> 8) / 16777216.0) * 4.0 - 2.0;
  }
  return a;
}

static void attn_case(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d, int threads) {
  unsigned st = (unsigned)(B * 1000 + H * 100 + Lq * 10 + Lk + d);
  double *q = rnd(B * H * Lq * d, &st), *k = rnd(B * H * Lk * d, &st), *v = rnd(B * H * Lk * d, &st);
  double *o = malloc((size_t)(B * H * Lq * d) * sizeof(double));
  double *o2 = malloc((size_t)(B * H * Lq * d) * sizeof(double));
  double *p = malloc((size_t)(B * H * Lq * Lk) * sizeof(double));
  CHECK(oracle_attn_f64(q, k, v, o, B, H, Lq, Lk, d, 0.5, threads) == 0);
  CHECK(oracle_attn_probs_f64(q, k, v, o2, p, B, H, Lq, Lk, d, 0.5) == 0);
  for (int64_t r = 0; r < B * H * Lq; ++r) {
    double s = 0.0;
    for (int64_t j = 0; j < Lk; ++j) s += p[r * Lk + j];
    CHECK(fabs(s - 1.0) < 1e-12);
  }
  for (int64_t i = 0; i < B * H * Lq * d; ++i) CHECK(o[i] == o2[i]);
  /* every row, in reverse order, through the row entry */
  const int64_t n = B * H * Lq;
  int64_t *rows = malloc((size_t)n * sizeof(int64_t));
  for (int64_t i = 0; i < n; ++i) rows[i] = n - 1 - i;
  double *orow = malloc((size_t)(n * d) * sizeof(double));
  CHECK(oracle_attn_rows_f64(q, k, v, B, H, Lq, Lk, d, 0.5, rows, n, orow, threads) == 0);
  for (int64_t i = 0; i < n; ++i)
    for (int64_t c = 0; c < d; ++c) CHECK(orow[i * d + c] == o[(n - 1 - i) * d + c]);
  /* argument checks: nothing is read or written */
  CHECK(oracle_attn_f64(NULL, k, v, o, B, H, Lq, Lk, d, 0.5, threads) != 0);
  CHECK(oracle_attn_f64(q, k, v, o, B, H, Lq, 0, d, 0.5, threads) != 0);
  CHECK(oracle_attn_f64(q, k, v, o, 0, H, Lq, Lk, d, 0.5, threads) != 0);
  rows[0] = n; /* out of range */
  CHECK(oracle_attn_rows_f64(q, k, v, B, H, Lq, Lk, d, 0.5, rows, n, orow, threads) != 0);
  rows[0] = -1;
  CHECK(oracle_attn_rows_f64(q, k, v, B, H, Lq, Lk, d, 0.5, rows, n, orow, threads) != 0);
  free(q); free(k); free(v); free(o); free(o2); free(p); free(rows); free(orow);
}

static void gn_case(int64_t N, int64_t C, int64_t S, int64_t G, int silu) {
  unsigned st = (unsigned)(N * 7 + C * 5 + S * 3 + G);
  double *x = rnd(N * C * S, &st), *g = rnd(C, &st), *b = rnd(C, &st);
  double *y = malloc((size_t)(N * C * S) * sizeof(double));
  CHECK(oracle_group_norm_f64(x, g, b, y, N, C, S, G, 1e-5, silu, 2) == 0);
  for (int64_t i = 0; i < N * C * S; ++i) CHECK(isfinite(y[i]));
  CHECK(oracle_group_norm_f64(x, g, b, y, N, C, S, 3, 1e-5, silu, 2) != 0 || C % 3 == 0);
  CHECK(oracle_group_norm_f64(NULL, g, b, y, N, C, S, G, 1e-5, silu, 2) != 0);
  CHECK(oracle_group_norm_f64(x, g, b, y, N, C, 0, G, 1e-5, silu, 2) != 0);
  free(x); free(g); free(b); free(y);
}

int main(void) {
  attn_case(1, 1, 1, 1, 1, 1);
  attn_case(2, 3, 5, 7, 8, 2);
  attn_case(1, 2, 33, 77, 40, 4);
  attn_case(2, 1, 3, 129, 24, 0);
  gn_case(1, 4, 8, 2, 0);
  gn_case(2, 12, 24, 4, 1);
  gn_case(3, 8, 64, 8, 1);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle sanitizer run: all checks passed\n");
  return 0;
}
