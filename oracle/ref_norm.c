/*
 * Reference oracle for forward row-wise normalization (LayerNorm, RMSNorm).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct CPU
 * definition that the GPU kernels are checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header, table or helper with the HIP library: it includes
 * only the C standard library and OpenMP.
 *
 * Every quantity is computed in IEEE float64 from the exact float32 inputs and
 * rounded once to float32 at the very end.  That follows the correctness
 * protocol of "RMSNorm on an RTX 5070: why more reduction threads did not win
 * every shape" (section "Correctness before timing"): the reference evaluates
 * the formula in float64 starting from the exact float32 values handed to the
 * device.
 *
 * Pins: tests/test_oracle_pins.py checks these functions against exact
 * rational brute force, closed forms, invariants and torch's float64 CPU
 * library routines; tests/test_negative_controls.py rebuilds this file with a
 * planted mistake (ORACLE_PLANT, below) and shows each one is caught.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

/* ORACLE_PLANT selects one deliberate mistake for the negative-control tests.
 * The shipped build leaves it at 0, where every planted line compiles away. */
#ifndef ORACLE_PLANT
#define ORACLE_PLANT 0
#endif

int oracle_max_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
int oracle_plant(void) { return ORACLE_PLANT; }

/*
 * LayerNorm forward, one row at a time.
 *
 * Statistics follow the equation in "Rewriting the layer norm and matmul
 * kernels", section "A reduction has to meet somewhere":
 *     mu_i      = (1/d) * sum_j x_ij
 *     sigma_i^2 = (1/d) * sum_j (x_ij - mu_i)^2        (biased, centered)
 * The normalised output applies the per-column scale and bias that the
 * kernels on "Field note 004: The load in flight, and the shape Triton uses"
 * load beside x, with eps inside the root:
 *     y_ij = (x_ij - mu_i) / sqrt(sigma_i^2 + eps) * gamma_j + beta_j
 * mean[i] = mu_i and rstd[i] = 1/sqrt(sigma_i^2 + eps) are optional outputs
 * (NULL skips them); mean64/var64 optionally expose the float64 statistics
 * before rounding, for the pins.
 *
 * x, y: row-major [rows, d] float32; gamma, beta: [d].  y may equal x.
 */
void oracle_layernorm_f64(const float *x, const float *gamma, const float *beta,
                          int64_t rows, int64_t d, float eps,
                          float *y, float *mean, float *rstd,
                          double *mean64, double *var64)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        const float *xi = x + i * d;
        float *yi = y + i * d;

        /* first reduction: the mean */
        double s = 0.0;
        for (int64_t j = 0; j < d; ++j)
            s += (double)xi[j];
        double mu = s / (double)d;

        /* second reduction: squared deviations around that mean */
        double q = 0.0;
        for (int64_t j = 0; j < d; ++j) {
            double c = (double)xi[j] - mu;
#if ORACLE_PLANT == 6
            c = (double)xi[j] + mu;              /* planted: wrong sign */
#endif
            q += c * c;
        }
        double var = q / (double)d;
#if ORACLE_PLANT == 3
        var = (d > 1) ? q / (double)(d - 1) : q; /* planted: unbiased variance */
#endif

        double rho = 1.0 / sqrt(var + (double)eps);
#if ORACLE_PLANT == 1
        rho = 1.0 / sqrt(var);                   /* planted: eps removed */
#endif
#if ORACLE_PLANT == 9
        rho = 1.0 / (sqrt(var) + (double)eps);   /* planted: eps outside the root */
#endif

        /* every x_ij is read before any y_ij is written, so y == x is safe */
        int64_t jend = d;
#if ORACLE_PLANT == 2
        jend = d - 1;                            /* planted: final column dropped */
#endif
        for (int64_t j = 0; j < jend; ++j) {
            double g = (double)gamma[j];
            double b = (double)beta[j];
#if ORACLE_PLANT == 4
            b = 0.0;                             /* planted: bias dropped */
#endif
#if ORACLE_PLANT == 5
            g = (double)gamma[i % d];            /* planted: scale indexed by row */
#endif
            yi[j] = (float)(((double)xi[j] - mu) * rho * g + b);
        }
        if (mean)   mean[i] = (float)mu;
        if (rstd)   rstd[i] = (float)rho;
        if (mean64) mean64[i] = mu;
        if (var64)  var64[i] = var;
    }
}

/*
 * RMSNorm forward, one row at a time, as the equation of "RMSNorm on an RTX
 * 5070" (section "The operator and the change") defines it:
 *     y_rc = x_rc * w_c * ( (1/D) * sum_j x_rj^2 + eps )^(-1/2)
 * rstd[r] = ((1/D) sum_j x_rj^2 + eps)^(-1/2) is optional (NULL skips it);
 * ms64 optionally exposes the float64 mean square.  y may equal x.
 */
void oracle_rmsnorm_f64(const float *x, const float *w,
                        int64_t rows, int64_t d, float eps,
                        float *y, float *rstd, double *ms64)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * d;
        float *yr = y + r * d;

        double s2 = 0.0;
        for (int64_t j = 0; j < d; ++j)
            s2 += (double)xr[j] * (double)xr[j];
        double ms = s2 / (double)d;
#if ORACLE_PLANT == 8
        ms = s2 / (double)(d + 1);               /* planted: wrong denominator */
#endif

        double rho = 1.0 / sqrt(ms + (double)eps);
#if ORACLE_PLANT == 7
        rho = 1.0 / sqrt(ms);                    /* planted: eps removed */
#endif

        for (int64_t c = 0; c < d; ++c)
            yr[c] = (float)((double)xr[c] * (double)w[c] * rho);
        if (rstd) rstd[r] = (float)rho;
        if (ms64) ms64[r] = ms;
    }
}

/*
 * Residual add fused before the normalization: h = x + r, then LayerNorm
 * (or RMSNorm) of h.  h is formed as a float32 addition, the precision of
 * the residual stream a caller stores, and the normalization above is then
 * applied to that rounded sum exactly as for a plain input.  h may be NULL.
 * y, h may equal x or r.
 */
void oracle_add_layernorm_f64(const float *x, const float *r, const float *gamma,
                              const float *beta, int64_t rows, int64_t d, float eps,
                              float *y, float *h, float *mean, float *rstd)
{
    #pragma omp parallel
    {
        /* the float32 sum of one row, kept before any output is written */
        float *hs = (float *)malloc((size_t)d * sizeof(float));
        #pragma omp for schedule(static)
        for (int64_t i = 0; i < rows; ++i) {
            const float *xi = x + i * d, *ri = r + i * d;
            float *yi = y + i * d;
            for (int64_t j = 0; j < d; ++j)
                hs[j] = xi[j] + ri[j];
#if ORACLE_PLANT == 10
            for (int64_t j = 0; j < d; ++j)
                hs[j] = xi[j];                   /* planted: residual dropped */
#endif

            double s = 0.0;
            for (int64_t j = 0; j < d; ++j)
                s += (double)hs[j];
            double mu = s / (double)d;
            double q = 0.0;
            for (int64_t j = 0; j < d; ++j) {
                double c = (double)hs[j] - mu;
                q += c * c;
            }
            double var = q / (double)d;
            double rho = 1.0 / sqrt(var + (double)eps);
            for (int64_t j = 0; j < d; ++j)
                yi[j] = (float)(((double)hs[j] - mu) * rho * (double)gamma[j] + (double)beta[j]);
            if (h)
                for (int64_t j = 0; j < d; ++j)
                    h[i * d + j] = hs[j];
            if (mean) mean[i] = (float)mu;
            if (rstd) rstd[i] = (float)rho;
        }
        free(hs);
    }
}

void oracle_add_rmsnorm_f64(const float *x, const float *r, const float *w,
                            int64_t rows, int64_t d, float eps,
                            float *y, float *h, float *rstd)
{
    #pragma omp parallel
    {
        float *hs = (float *)malloc((size_t)d * sizeof(float));
        #pragma omp for schedule(static)
        for (int64_t i = 0; i < rows; ++i) {
            const float *xi = x + i * d, *ri = r + i * d;
            float *yi = y + i * d;
            for (int64_t j = 0; j < d; ++j)
                hs[j] = xi[j] + ri[j];
#if ORACLE_PLANT == 11
            for (int64_t j = 0; j < d; ++j)
                hs[j] = ri[j];                   /* planted: input dropped */
#endif

            double s2 = 0.0;
            for (int64_t j = 0; j < d; ++j)
                s2 += (double)hs[j] * (double)hs[j];
            double rho = 1.0 / sqrt(s2 / (double)d + (double)eps);
            for (int64_t j = 0; j < d; ++j)
                yi[j] = (float)((double)hs[j] * (double)w[j] * rho);
            if (h)
                for (int64_t j = 0; j < d; ++j)
                    h[i * d + j] = hs[j];
            if (rstd) rstd[i] = (float)rho;
        }
        free(hs);
    }
}
