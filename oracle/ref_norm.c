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
 * before rounding, for the pins, and y64 the float64 outputs before their one
 * rounding (what a narrower storage format is rounded from).
 *
 * x, y: row-major [rows, d] float32; gamma, beta: [d].  y may equal x.
 */
void oracle_layernorm_f64(const float *x, const float *gamma, const float *beta,
                          int64_t rows, int64_t d, float eps,
                          float *y, float *mean, float *rstd,
                          double *mean64, double *var64, double *y64)
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
            const double v = ((double)xi[j] - mu) * rho * g + b;
            yi[j] = (float)v;
            if (y64) y64[i * d + j] = v;
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
 * ms64 optionally exposes the float64 mean square and y64 the float64
 * outputs before rounding.  y may equal x.
 */
void oracle_rmsnorm_f64(const float *x, const float *w,
                        int64_t rows, int64_t d, float eps,
                        float *y, float *rstd, double *ms64, double *y64)
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

        for (int64_t c = 0; c < d; ++c) {
            const double v = (double)xr[c] * (double)w[c] * rho;
            yr[c] = (float)v;
            if (y64) y64[r * d + c] = v;
        }
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

/*
 * 16-bit storage formats: IEEE binary16 (fmt 1) and bfloat16 (fmt 2).
 *
 * A format is (p significand bits including the implicit one, emin, emax):
 * binary16 (11, -14, 15), bfloat16 (8, -126, 127).  A finite value is
 * (-1)^s * m * 2^(e - p + 1) with integer m < 2^p, and e = emin for the
 * subnormals.  Widening is exact (every such value is a float32, hence a
 * float64); narrowing rounds a float64 once, to nearest with ties to even, as
 * IEEE 754 defines for a conversion to a narrower format: values at or past
 * the overflow midpoint become infinities.
 *
 * The normalization over 16-bit storage is then: widen the inputs exactly,
 * apply the float64 definition above, round each output once from its float64
 * value.  The fused residual sum h = x + r is rounded to the storage format
 * once, from the exact sum, and the norm is applied to that stored h.
 */
static void fmt16(int fmt, int *p, int *emin, int *emax)
{
    if (fmt == 1) { *p = 11; *emin = -14;  *emax = 15;  }
    else          { *p = 8;  *emin = -126; *emax = 127; }
}

double oracle_widen16(uint16_t b, int fmt)
{
    int p, emin, emax;
    fmt16(fmt, &p, &emin, &emax);
    const int mbits = p - 1;                       /* stored fraction bits */
    const int ebits = 15 - mbits;
    const int bias = emax;
    const int s = b >> 15;
    const int ef = (b >> mbits) & ((1 << ebits) - 1);
    const int mf = b & ((1 << mbits) - 1);
    double v;
    if (ef == (1 << ebits) - 1)                    /* infinity or NaN */
        v = mf ? NAN : INFINITY;
    else if (ef == 0)                              /* zero or subnormal */
        v = ldexp((double)mf, emin - mbits);
    else
        v = ldexp((double)((1 << mbits) | mf), ef - bias - mbits);
    return s ? -v : v;
}

uint16_t oracle_round16(double v, int fmt)
{
    int p, emin, emax;
    fmt16(fmt, &p, &emin, &emax);
    const int mbits = p - 1;
    const int ebits = 15 - mbits;
    const uint16_t sign = signbit(v) ? 0x8000u : 0u;
    const uint16_t inf = (uint16_t)(((1u << ebits) - 1u) << mbits);
    if (isnan(v)) return (uint16_t)(sign | inf | (1u << (mbits - 1)));
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | inf);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                                  /* a = f * 2^e, 0.5 <= f < 1 */
    int E = e - 1;                                 /* floor(log2 a) */
    if (E < emin) E = emin;                        /* the subnormal quantum */
    /* a / 2^(E - mbits) is exact (a power-of-two scaling); round that to an
       integer, ties to even (the default rounding mode of nearbyint) */
    double m = nearbyint(ldexp(a, mbits - E));
#if ORACLE_PLANT == 12
    m = floor(ldexp(a, mbits - E));                /* planted: truncation */
#endif
#if ORACLE_PLANT == 13
    m = round(ldexp(a, mbits - E));                /* planted: ties away from zero */
#endif
    if (m >= (double)(1 << p)) {                   /* carried into the next binade */
        m /= 2.0;
        E += 1;
    }
    if (E > emax) return (uint16_t)(sign | inf);   /* overflow */
    if (m < (double)(1 << mbits))                  /* subnormal (E == emin) */
        return (uint16_t)(sign | (uint16_t)m);
    return (uint16_t)(sign | (uint16_t)((E + emax) << mbits) | ((uint16_t)m & ((1u << mbits) - 1u)));
}

void oracle_widen16_n(const uint16_t *in, int fmt, int64_t n, float *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)oracle_widen16(in[i], fmt);
}

void oracle_round16_n(const double *in, int fmt, int64_t n, uint16_t *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_round16(in[i], fmt);
}

/* h = x + r in the storage format.  The float64 sum of two 16-bit values is
 * exact unless their exponents differ by more than 45 (possible for bfloat16
 * only); then the smaller addend is below 2^-38 of an ulp of the larger, no
 * rounding midpoint is near, and rounding the float64 sum gives what rounding
 * the exact sum gives: the larger addend. */
void oracle_add16_n(const uint16_t *x, const uint16_t *r, int fmt, int64_t n, uint16_t *h)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double s = oracle_widen16(x[i], fmt) + oracle_widen16(r[i], fmt);
#if ORACLE_PLANT == 14
        s = oracle_widen16(x[i], fmt);             /* planted: residual dropped */
#endif
        h[i] = oracle_round16(s, fmt);
    }
}

/*
 * Backward of the two normalizations: the exact derivative of the definitions
 * above with respect to x and to the per-column parameters, given the
 * upstream gradient dy and the per-row statistics the forward returned
 * (taken as inputs, as a training step passes them from forward to backward).
 *
 * LayerNorm, per row i, with xhat_ij = (x_ij - mu_i) * rho_i and
 * g_ij = dy_ij * gamma_j:
 *     dx_ij    = rho_i * (g_ij - (1/d) sum_k g_ik - xhat_ij * (1/d) sum_k g_ik xhat_ik)
 *     dgamma_j = sum_i dy_ij * xhat_ij,     dbeta_j = sum_i dy_ij
 * (differentiating y = xhat * gamma + beta through mu and rho: d mu/d x_k = 1/d
 * and d rho/d x_k = -rho^3 (x_k - mu) / d.)
 *
 * RMSNorm, per row i, with xhat_ij = x_ij * rho_i and g_ij = dy_ij * w_j:
 *     dx_ij = rho_i * (g_ij - xhat_ij * (1/d) sum_k g_ik xhat_ik),   dw_j = sum_i dy_ij xhat_ij
 *
 * The statistics come in as float64 (the forward's float32 values widened,
 * or exact ones for the pins).  Everything is float64 from the float32
 * inputs; dx is rounded once to
 * float32 (dx64 optionally keeps it unrounded), the parameter gradients
 * likewise (dg64/db64 unrounded).  dxs64 optionally receives, per element,
 * rho_i * (|g_ij| + mean_k |g_ik| + |xhat_ij| * mean_k |g_ik xhat_ik|)
 * (RMSNorm without the middle term): the magnitudes a float32 evaluation of
 * dx carries rounding error in proportion to.  adg64/adb64 optionally receive
 * sum_i |dy_ij xhat_ij| and sum_i |dy_ij|, the magnitudes a float32 column
 * sum's rounding error scales with.  Any optional output may be NULL.
 */
void oracle_layernorm_bwd_f64(const float *dy, const float *x, const float *gamma,
                              const double *mean, const double *rstd, int64_t rows, int64_t d,
                              float *dx, double *dx64, double *dxs64, float *dgamma, float *dbeta,
                              double *dg64, double *db64, double *adg64, double *adb64)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        const float *xi = x + i * d, *dyi = dy + i * d;
        const double mu = mean[i], rho = rstd[i];
        double s1 = 0.0, s2 = 0.0, a1 = 0.0, a2 = 0.0;
        for (int64_t k = 0; k < d; ++k) {
            const double xh = ((double)xi[k] - mu) * rho;
            const double g = (double)dyi[k] * (double)gamma[k];
            s1 += g;
            s2 += g * xh;
            a1 += fabs(g);
            a2 += fabs(g * xh);
        }
        const double m1 = s1 / (double)d, m2 = s2 / (double)d;
        const double am1 = a1 / (double)d, am2 = a2 / (double)d;
        for (int64_t j = 0; j < d; ++j) {
            const double xh = ((double)xi[j] - mu) * rho;
            const double g = (double)dyi[j] * (double)gamma[j];
            double v = rho * (g - m1 - xh * m2);
#if ORACLE_PLANT == 15
            v = rho * (g - xh * m2);                 /* planted: mean of g dropped */
#endif
#if ORACLE_PLANT == 16
            v = rho * (g - m1 + xh * m2);            /* planted: sign of the projection */
#endif
            if (dx) dx[i * d + j] = (float)v;
            if (dx64) dx64[i * d + j] = v;
            if (dxs64) dxs64[i * d + j] = rho * (fabs(g) + am1 + fabs(xh) * am2);
        }
    }
    /* column sums, rows in ascending order */
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < d; ++j) {
        double sg = 0.0, sb = 0.0, ag = 0.0, ab = 0.0;
        for (int64_t i = 0; i < rows; ++i) {
            const double dyv = (double)dy[i * d + j];
            double xh = ((double)x[i * d + j] - mean[i]) * rstd[i];
#if ORACLE_PLANT == 17
            xh = (double)x[i * d + j] * rstd[i];           /* planted: mean not removed in dgamma */
#endif
            sg += dyv * xh;
            sb += dyv;
            ag += fabs(dyv * xh);
            ab += fabs(dyv);
        }
        if (dgamma) dgamma[j] = (float)sg;
        if (dbeta) dbeta[j] = (float)sb;
        if (dg64) dg64[j] = sg;
        if (db64) db64[j] = sb;
        if (adg64) adg64[j] = ag;
        if (adb64) adb64[j] = ab;
    }
}

void oracle_rmsnorm_bwd_f64(const float *dy, const float *x, const float *w, const double *rstd,
                            int64_t rows, int64_t d, float *dx, double *dx64, double *dxs64, float *dw,
                            double *dw64, double *adw64)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        const float *xi = x + i * d, *dyi = dy + i * d;
        const double rho = rstd[i];
        double s2 = 0.0, a2 = 0.0;
        for (int64_t k = 0; k < d; ++k) {
            const double t = (double)dyi[k] * (double)w[k] * ((double)xi[k] * rho);
            s2 += t;
            a2 += fabs(t);
        }
        const double m2 = s2 / (double)d, am2 = a2 / (double)d;
        for (int64_t j = 0; j < d; ++j) {
            const double xh = (double)xi[j] * rho;
            const double g = (double)dyi[j] * (double)w[j];
            double v = rho * (g - xh * m2);
#if ORACLE_PLANT == 18
            v = g - xh * m2;                         /* planted: outer rho dropped */
#endif
            if (dx) dx[i * d + j] = (float)v;
            if (dx64) dx64[i * d + j] = v;
            if (dxs64) dxs64[i * d + j] = rho * (fabs(g) + fabs(xh) * am2);
        }
    }
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < d; ++j) {
        double s = 0.0, a = 0.0;
        for (int64_t i = 0; i < rows; ++i) {
            const double t = (double)dy[i * d + j] * ((double)x[i * d + j] * rstd[i]);
            s += t;
            a += fabs(t);
        }
        if (dw) dw[j] = (float)s;
        if (dw64) dw64[j] = s;
        if (adw64) adw64[j] = a;
    }
}
