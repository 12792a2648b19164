/*
 * attn_oracle.c -- plain fp64 CPU oracle for scaled dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes.  The page "Diffusion inference engine from scratch:
 * Rust + wgpu" (ybb.press), section 3.2 (the Flash-Attention-equivalent
 * cross-attention kernel), describes attention whose queries come from the
 * latent feature map and whose keys/values come from the text context, and
 * whose result is the softmax-weighted sum of values over the Q.K^T scores.
 * The blockwise online-softmax recurrence sketched there is only a faster
 * way to reach the same numbers, so this oracle is the plain definition,
 * written out step by step for every batch b, head h and query row i:
 *
 *   1. s_j   = sigma * sum_c q[b,h,i,c] * k[b,h,j,c]        (score row)
 *   2. m     = max_j s_j
 *   3. e_j   = exp(s_j - m)
 *   4. l     = sum_j e_j
 *   5. p_j   = e_j / l                                       (softmax row)
 *   6. o[c]  = sum_j p_j * v[b,h,j,c]
 *
 * sigma is the caller's scale (1/sqrt(d) for the UNet's attention), applied
 * to the scores, never folded into Q.  All arithmetic is IEEE double with
 * sequential summation in index order; the file must be built without
 * -ffast-math so the result is deterministic.  Tensors are contiguous
 * [B, H, L, d] arrays of double (the caller widens bf16/fp32 inputs exactly).
 *
 * Rows are independent, so the only parallelism is an OpenMP loop over
 * (b, h, i); it does not change any result.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

/* Steps 1-6 for one query row.  s is caller scratch of Lk doubles; when
 * p_out is non-NULL the normalised softmax row (step 5) is also returned. */
static void attend_row(const double *q_row, const double *k_bh,
                       const double *v_bh, int64_t Lk, int64_t d, double sigma,
                       double *s, double *o_row, double *p_out) {
  /* 1. scores */
  for (int64_t j = 0; j < Lk; ++j) {
    const double *k_row = k_bh + j * d;
    double dot = 0.0;
    for (int64_t c = 0; c < d; ++c) dot += q_row[c] * k_row[c];
    s[j] = sigma * dot;
  }
  /* 2. row maximum */
  double m = s[0];
  for (int64_t j = 1; j < Lk; ++j)
    if (s[j] > m) m = s[j];
  /* 3-4. exponentials and their sum */
  double l = 0.0;
  for (int64_t j = 0; j < Lk; ++j) {
    s[j] = exp(s[j] - m);
    l += s[j];
  }
  /* 5. normalise */
  for (int64_t j = 0; j < Lk; ++j) s[j] = s[j] / l;
  if (p_out)
    for (int64_t j = 0; j < Lk; ++j) p_out[j] = s[j];
  /* 6. weighted sum of value rows */
  for (int64_t c = 0; c < d; ++c) o_row[c] = 0.0;
  for (int64_t j = 0; j < Lk; ++j) {
    const double *v_row = v_bh + j * d;
    const double pj = s[j];
    for (int64_t c = 0; c < d; ++c) o_row[c] += pj * v_row[c];
  }
}

static int check_dims(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d) {
  return (B < 1 || H < 1 || Lq < 1 || Lk < 1 || d < 1) ? ORACLE_EINVAL : ORACLE_OK;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

/* Number of threads an OpenMP region would use (1 without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Full attention: out[B,H,Lq,d] for every row.  nthreads <= 0 keeps the
 * OpenMP default. */
int oracle_attn_f64(const double *q, const double *k, const double *v,
                    double *out, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                    int64_t d, double scale, int nthreads) {
  if (!q || !k || !v || !out) return ORACLE_EINVAL;
  if (check_dims(B, H, Lq, Lk, d)) return ORACLE_EINVAL;
  set_threads(nthreads);
  const int64_t rows = B * H * Lq;
  int failed = 0;
#pragma omp parallel
  {
    double *s = (double *)malloc((size_t)Lk * sizeof(double));
    if (!s) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; ++r) {
      if (!s) continue;
      const int64_t bh = r / Lq;
      attend_row(q + r * d, k + bh * Lk * d, v + bh * Lk * d, Lk, d, scale, s,
                 out + r * d, NULL);
    }
    free(s);
  }
  return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/* Selected rows only: rows[n] is the flattened index (b*H + h)*Lq + i, and
 * out is [nrows, d].  Used for sampled parity checks at sizes where the
 * full oracle would take too long. */
int oracle_attn_rows_f64(const double *q, const double *k, const double *v,
                         int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                         int64_t d, double scale, const int64_t *rows,
                         int64_t nrows, double *out, int nthreads) {
  if (!q || !k || !v || !out || (!rows && nrows > 0) || nrows < 0)
    return ORACLE_EINVAL;
  if (check_dims(B, H, Lq, Lk, d)) return ORACLE_EINVAL;
  const int64_t total = B * H * Lq;
  for (int64_t n = 0; n < nrows; ++n)
    if (rows[n] < 0 || rows[n] >= total) return ORACLE_EINVAL;
  set_threads(nthreads);
  int failed = 0;
#pragma omp parallel
  {
    double *s = (double *)malloc((size_t)Lk * sizeof(double));
    if (!s) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t n = 0; n < nrows; ++n) {
      if (!s) continue;
      const int64_t r = rows[n];
      const int64_t bh = r / Lq;
      attend_row(q + r * d, k + bh * Lk * d, v + bh * Lk * d, Lk, d, scale, s,
                 out + n * d, NULL);
    }
    free(s);
  }
  return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/* Softmax matrix P[B,H,Lq,Lk] (step 5) next to the output, for small cases
 * such as the rows-sum-to-one check. */
int oracle_attn_probs_f64(const double *q, const double *k, const double *v,
                          double *out, double *probs, int64_t B, int64_t H,
                          int64_t Lq, int64_t Lk, int64_t d, double scale) {
  if (!q || !k || !v || !out || !probs) return ORACLE_EINVAL;
  if (check_dims(B, H, Lq, Lk, d)) return ORACLE_EINVAL;
  double *s = (double *)malloc((size_t)Lk * sizeof(double));
  if (!s) return ORACLE_ENOMEM;
  const int64_t rows = B * H * Lq;
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t bh = r / Lq;
    attend_row(q + r * d, k + bh * Lk * d, v + bh * Lk * d, Lk, d, scale, s,
               out + r * d, probs + r * Lk);
  }
  free(s);
  return ORACLE_OK;
}
