/*
 * group_norm_oracle.c -- plain fp64 CPU oracle for GroupNorm, optionally
 * followed by SiLU.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes.  The page "Diffusion inference engine from scratch:
 * Rust + wgpu" (ybb.press), section 3.1, normalises the UNet's activations
 * group by group: each group's mean and variance (the page writes the
 * variance as the mean of squares minus the squared mean) give an inverse
 * standard deviation 1/sqrt(var + eps); the page's model-level list of
 * fusions pairs this GroupNorm with the SiLU that follows it.  For an
 * activation x laid out as contiguous [N, C, S] (S = H*W positions per
 * channel) and G groups of C/G consecutive channels, for every sample n and
 * group g, with M = (C/G)*S elements:
 *
 *   1. mu    = (1/M) sum x                      over the group's elements
 *   2. var   = (1/M) sum (x - mu)^2              (population variance; equal
 *                                                 to E[x^2] - mu^2, written in
 *                                                 the two-pass form)
 *   3. y     = (x - mu) / sqrt(var + eps) * gamma[c] + beta[c]
 *   4. silu: y = y / (1 + exp(-y))               (only when silu != 0)
 *
 * All arithmetic is IEEE double with sequential sums in index order; build
 * without -ffast-math.  Groups are independent; the OpenMP loop over
 * (n, g) does not change any result.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL 1

static void norm_group(const double *xg, double *yg, const double *gamma,
                       const double *beta, int64_t c0, int64_t cpg, int64_t S,
                       double eps, int silu) {
  const int64_t M = cpg * S;
  /* 1. mean */
  double sum = 0.0;
  for (int64_t i = 0; i < M; ++i) sum += xg[i];
  const double mu = sum / (double)M;
  /* 2. variance about the mean */
  double ss = 0.0;
  for (int64_t i = 0; i < M; ++i) {
    const double t = xg[i] - mu;
    ss += t * t;
  }
  const double var = ss / (double)M;
  const double inv_std = 1.0 / sqrt(var + eps);
  /* 3. normalise, per-channel affine; 4. SiLU */
  for (int64_t cc = 0; cc < cpg; ++cc) {
    const double ga = gamma[c0 + cc], be = beta[c0 + cc];
    for (int64_t s = 0; s < S; ++s) {
      const int64_t i = cc * S + s;
      double y = (xg[i] - mu) * inv_std * ga + be;
      if (silu) y = y / (1.0 + exp(-y));
      yg[i] = y;
    }
  }
}

/* x, y: [N, C, S] contiguous; gamma, beta: [C]. */
int oracle_group_norm_f64(const double *x, const double *gamma, const double *beta,
                          double *y, int64_t N, int64_t C, int64_t S, int64_t G,
                          double eps, int silu, int nthreads) {
  if (!x || !gamma || !beta || !y || N < 1 || C < 1 || S < 1 || G < 1 || C % G != 0)
    return ORACLE_EINVAL;
  const int64_t cpg = C / G;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t ng = 0; ng < N * G; ++ng) {
    const int64_t n = ng / G, g = ng % G;
    const int64_t off = (n * C + g * cpg) * S;
    norm_group(x + off, y + off, gamma, beta, g * cpg, cpg, S, eps, silu);
  }
  (void)nthreads;
  return ORACLE_OK;
}
