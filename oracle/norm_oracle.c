/*
 * norm_oracle.c -- plain fp64 CPU oracle for the LayerNorm / RMSNorm backward.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The GPU path never calls it and
 * shares no code, header or constant with it.
 *
 * Everything here is the textbook definition written out loop by loop in
 * IEEE double precision (built with -ffp-contract=off, so no fused
 * multiply-add), with every sum taken in ascending index order. Inputs are
 * fp64 arrays; callers widen the exact bits the GPU received.
 *
 * Notation follows "Norm backward in Triton -- the dγ/dβ reduction", section
 * "The gradients (the half-page you reverse)": per row x of width N with saved
 * statistics (mean, rstd = 1/sigma), xhat = (x - mean) * rstd, dyhat = dy*gamma,
 *
 *   dx     = rstd * (dyhat - mean_j(dyhat) - xhat * mean_j(dyhat * xhat))
 *   dgamma = sum over rows of dy * xhat
 *   dbeta  = sum over rows of dy
 *
 * and RMSNorm has no mean: xhat = x * rstd with rstd = 1/sqrt(mean(x^2)+eps),
 * and its dx has no mean_j(dyhat) term. "05: Layer norm" (the Phobos
 * tutorial) states the same dx with its two row means named the other way
 * round and the terms grouped differently (its ln_bwd_dx), and the same
 * dgamma/dbeta over xhat recomputed from the saved statistics (ln_bwd_dwdb).
 *
 * kind: 0 = LayerNorm, 1 = RMSNorm (this file's own convention).
 */
#include <math.h>
#include <stddef.h>

#define ORACLE_LAYERNORM 0
#define ORACLE_RMSNORM 1

/*
 * Forward statistics, as the forward pass would save them.
 * LayerNorm ("05: Layer norm", ln_fwd): mean = sum(x)/N,
 *   var = sum((x-mean)^2)/N (biased, two passes), rstd = 1/sqrt(var+eps).
 * RMSNorm ("Norm backward in Triton", "The gradients"):
 *   rstd = 1/sqrt(sum(x^2)/N + eps); mean (if given) is set to 0.
 */
void oracle_norm_fwd_stats(int kind, const double *x, long M, long N,
                           double eps, double *mean, double *rstd)
{
    for (long r = 0; r < M; ++r) {
        const double *xr = x + r * N;
        if (kind == ORACLE_LAYERNORM) {
            double s = 0.0;
            for (long j = 0; j < N; ++j)
                s += xr[j];
            double mu = s / (double)N;
            double v = 0.0;
            for (long j = 0; j < N; ++j) {
                double d = xr[j] - mu;
                v += d * d;
            }
            v = v / (double)N;
            mean[r] = mu;
            rstd[r] = 1.0 / sqrt(v + eps);
        } else {
            double q = 0.0;
            for (long j = 0; j < N; ++j)
                q += xr[j] * xr[j];
            if (mean)
                mean[r] = 0.0;
            rstd[r] = 1.0 / sqrt(q / (double)N + eps);
        }
    }
}

/*
 * Forward output y = gamma * xhat + beta (beta may be NULL: treated as 0),
 * also returning the statistics ("05: Layer norm", the Phobos tutorial's
 * forward). The reference for the GPU forward, and the function whose finite
 * differences of L = sum(dy * y) pin the backward.
 */
void oracle_norm_fwd(int kind, const double *x, const double *gamma,
                     const double *beta, long M, long N, double eps,
                     double *y, double *mean, double *rstd)
{
    oracle_norm_fwd_stats(kind, x, M, N, eps, mean, rstd);
    for (long r = 0; r < M; ++r) {
        double mu = (kind == ORACLE_LAYERNORM) ? mean[r] : 0.0;
        double rs = rstd[r];
        for (long j = 0; j < N; ++j) {
            double xh = (x[r * N + j] - mu) * rs;
            double b = beta ? beta[j] : 0.0;
            y[r * N + j] = gamma[j] * xh + b;
        }
    }
}

/*
 * Input gradient, row by row ("The gradients": dx is per row and needs two
 * in-row means; RMSNorm drops the first). mean may be NULL for RMSNorm.
 */
void oracle_norm_bwd_dx(int kind, const double *x, const double *dy,
                        const double *gamma, const double *mean,
                        const double *rstd, long M, long N, double *dx)
{
    for (long r = 0; r < M; ++r) {
        const double *xr = x + r * N;
        const double *dyr = dy + r * N;
        double mu = (kind == ORACLE_LAYERNORM) ? mean[r] : 0.0;
        double rs = rstd[r];

        double sum_dyhat = 0.0;       /* sum_j dyhat_j          */
        double sum_dyhat_xhat = 0.0;  /* sum_j dyhat_j * xhat_j */
        for (long j = 0; j < N; ++j) {
            double xh = (xr[j] - mu) * rs;
            double dyh = dyr[j] * gamma[j];
            sum_dyhat += dyh;
            sum_dyhat_xhat += dyh * xh;
        }
        double mean_dyhat = (kind == ORACLE_LAYERNORM) ? sum_dyhat / (double)N : 0.0;
        double mean_dyhat_xhat = sum_dyhat_xhat / (double)N;

        for (long j = 0; j < N; ++j) {
            double xh = (xr[j] - mu) * rs;
            double dyh = dyr[j] * gamma[j];
            dx[r * N + j] = rs * (dyh - mean_dyhat - xh * mean_dyhat_xhat);
        }
    }
}

/*
 * Weight gradients, summed over every row in ascending row order
 * ("Norm & activation backward", "Half two: dγ and dβ reduce across the whole
 * batch"): dgamma_j = sum_r dy_rj * xhat_rj, dbeta_j = sum_r dy_rj.
 * dbeta may be NULL. M = 0 gives zeros (the empty sum).
 */
void oracle_norm_bwd_wgrad(int kind, const double *x, const double *dy,
                           const double *mean, const double *rstd, long M,
                           long N, double *dgamma, double *dbeta)
{
    for (long j = 0; j < N; ++j) {
        dgamma[j] = 0.0;
        if (dbeta)
            dbeta[j] = 0.0;
    }
    for (long r = 0; r < M; ++r) {
        double mu = (kind == ORACLE_LAYERNORM) ? mean[r] : 0.0;
        double rs = rstd[r];
        for (long j = 0; j < N; ++j) {
            double xh = (x[r * N + j] - mu) * rs;
            dgamma[j] += dy[r * N + j] * xh;
            if (dbeta)
                dbeta[j] += dy[r * N + j];
        }
    }
}
