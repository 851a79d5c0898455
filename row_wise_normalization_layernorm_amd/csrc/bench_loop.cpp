// bench_loop.cpp — libmi_norm_bench.so: native timing loops for bench.py.
//
// Host code only.  Each step is one full call of the public C ABI
// (validation, dispatch, one kernel launch) on one buffer set; step s uses set
// s % nsets so that, with enough sets, every step reads x that has left the
// caches.  Issuing the calls from C keeps the GPU fed: a Python-level call
// costs more than a kernel of a few microseconds.
#include <cstdint>

#include "mi_norm_tuning.h"

extern "C" {

// LayerNorm: xs/ys/means/rstds are arrays of nsets device pointers
// (means/rstds may be NULL, or hold NULL entries).  variant < 0 uses the
// dispatcher.  Returns the first non-OK status, else MI_NORM_OK.
int mi_bench_layernorm_loop(const float *const *xs, const float *gamma, const float *beta,
                            float *const *ys, float *const *means, float *const *rstds, int nsets,
                            int64_t rows, int64_t d, float eps, int steps, int variant,
                            hipStream_t stream) {
    for (int s = 0; s < steps; ++s) {
        const int k = s % nsets;
        float *m = means ? means[k] : nullptr;
        float *r = rstds ? rstds[k] : nullptr;
        const mi_norm_status st =
            variant < 0 ? mi_layernorm_fwd(xs[k], gamma, beta, ys[k], rows, d, eps, m, r, stream)
                        : mi_layernorm_fwd_variant(variant, xs[k], gamma, beta, ys[k], rows, d, eps, m,
                                                   r, stream);
        if (st != MI_NORM_OK) return st;
    }
    return MI_NORM_OK;
}

int mi_bench_rmsnorm_loop(const float *const *xs, const float *w, float *const *ys,
                          float *const *rstds, int nsets, int64_t rows, int64_t d, float eps, int steps,
                          int variant, hipStream_t stream) {
    for (int s = 0; s < steps; ++s) {
        const int k = s % nsets;
        float *r = rstds ? rstds[k] : nullptr;
        const mi_norm_status st =
            variant < 0 ? mi_rmsnorm_fwd(xs[k], w, ys[k], rows, d, eps, r, stream)
                        : mi_rmsnorm_fwd_variant(variant, xs[k], w, ys[k], rows, d, eps, r, stream);
        if (st != MI_NORM_OK) return st;
    }
    return MI_NORM_OK;
}

// Residual add + LayerNorm / RMSNorm: rs[k] the residual, hs[k] where x + r is
// written (hs or its entries may be NULL).
int mi_bench_add_layernorm_loop(const float *const *xs, const float *const *rs, const float *gamma,
                                const float *beta, float *const *ys, float *const *hs,
                                float *const *means, float *const *rstds, int nsets, int64_t rows,
                                int64_t d, float eps, int steps, int variant, hipStream_t stream) {
    for (int s = 0; s < steps; ++s) {
        const int k = s % nsets;
        float *h = hs ? hs[k] : nullptr;
        float *m = means ? means[k] : nullptr;
        float *r = rstds ? rstds[k] : nullptr;
        const mi_norm_status st =
            variant < 0 ? mi_add_layernorm_fwd(xs[k], rs[k], gamma, beta, ys[k], h, rows, d, eps, m, r, stream)
                        : mi_add_layernorm_fwd_variant(variant, xs[k], rs[k], gamma, beta, ys[k], h, rows, d,
                                                       eps, m, r, stream);
        if (st != MI_NORM_OK) return st;
    }
    return MI_NORM_OK;
}

int mi_bench_add_rmsnorm_loop(const float *const *xs, const float *const *rs, const float *w,
                              float *const *ys, float *const *hs, float *const *rstds, int nsets,
                              int64_t rows, int64_t d, float eps, int steps, int variant,
                              hipStream_t stream) {
    for (int s = 0; s < steps; ++s) {
        const int k = s % nsets;
        float *h = hs ? hs[k] : nullptr;
        float *r = rstds ? rstds[k] : nullptr;
        const mi_norm_status st =
            variant < 0 ? mi_add_rmsnorm_fwd(xs[k], rs[k], w, ys[k], h, rows, d, eps, r, stream)
                        : mi_add_rmsnorm_fwd_variant(variant, xs[k], rs[k], w, ys[k], h, rows, d, eps, r,
                                                     stream);
        if (st != MI_NORM_OK) return st;
    }
    return MI_NORM_OK;
}

// Any operation, storage type and row strides through mi_norm_fwd: *base
// holds everything but the per-set row and statistics pointers (rs, hs,
// means, rstds may be NULL).
int mi_bench_norm_loop(const mi_norm_problem *base, const void *const *xs, const void *const *rs,
                       void *const *ys, void *const *hs, float *const *means, float *const *rstds,
                       int nsets, int steps, int variant, hipStream_t stream) {
    mi_norm_problem p = *base;
    for (int s = 0; s < steps; ++s) {
        const int k = s % nsets;
        p.x = xs[k];
        p.r = rs ? rs[k] : nullptr;
        p.y = ys[k];
        p.h = hs ? hs[k] : nullptr;
        p.mean = means ? means[k] : nullptr;
        p.rstd = rstds ? rstds[k] : nullptr;
        const mi_norm_status st = variant < 0 ? mi_norm_fwd(&p, stream) : mi_norm_fwd_variant(variant, &p, stream);
        if (st != MI_NORM_OK) return st;
    }
    return MI_NORM_OK;
}

// Backward: *base holds everything but the per-set pointers (dgs, dbs may
// be NULL or hold NULL entries); the workspace in *base serves every step.
int mi_bench_bwd_loop(const mi_norm_bwd_problem *base, const void *const *dys, const void *const *xs,
                      void *const *dxs, const float *const *means, const float *const *rstds,
                      float *const *dgs, float *const *dbs, int nsets, int steps, int variant,
                      hipStream_t stream) {
    mi_norm_bwd_problem p = *base;
    for (int s = 0; s < steps; ++s) {
        const int k = s % nsets;
        p.dy = dys[k];
        p.x = xs[k];
        p.dx = dxs[k];
        p.mean = means ? means[k] : nullptr;
        p.rstd = rstds[k];
        p.dparams0 = dgs ? dgs[k] : nullptr;
        p.dparams1 = dbs ? dbs[k] : nullptr;
        const mi_norm_status st = variant < 0 ? mi_norm_bwd(&p, stream) : mi_norm_bwd_variant(variant, &p, stream);
        if (st != MI_NORM_OK) return st;
    }
    return MI_NORM_OK;
}

int mi_bench_copy_loop(const float *const *srcs, float *const *dsts, int nsets, int64_t n, int steps,
                       hipStream_t stream) {
    for (int s = 0; s < steps; ++s) {
        const int k = s % nsets;
        const mi_norm_status st = mi_copy_f32(srcs[k], dsts[k], n, stream);
        if (st != MI_NORM_OK) return st;
    }
    return MI_NORM_OK;
}

// The calibration launches of mi_calib_launch: kind 0 empty, 1 read srcs[k],
// 2 write dsts[k] (n float32 each).
int mi_bench_calib_loop(int kind, const float *const *srcs, float *const *dsts, int nsets, int64_t n,
                        int steps, hipStream_t stream) {
    for (int s = 0; s < steps; ++s) {
        const int k = s % nsets;
        const mi_norm_status st =
            mi_calib_launch(kind, srcs ? srcs[k] : nullptr, dsts ? dsts[k] : nullptr, n, stream);
        if (st != MI_NORM_OK) return st;
    }
    return MI_NORM_OK;
}

}  // extern "C"
