/*
 * mi_norm_tuning.h — the variant table, forced-variant calls and calibration
 * kernels of libmi_norm.so, for tests and benchmarks.
 *
 * libmi_norm.so exports these beside the calls of mi_norm.h, but they are
 * not part of its public interface: they expose how the library is tuned
 * (which compiled kernel shapes exist and which one a problem gets), which
 * may change from one build to the next.  Applications include mi_norm.h
 * only.  Every call here follows mi_norm.h's conventions and error rules.
 */
#ifndef MI_NORM_TUNING_H
#define MI_NORM_TUNING_H

#include "mi_norm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------------------
 * Kernel variants.  Every call of mi_norm.h is served by one compiled kernel variant
 * chosen from the operation, the storage type, the row width d, the pointer
 * alignment and strides, and the row count.  The calls below expose that
 * table so tests can drive every variant and benchmarks can compare them.
 * They follow the same conventions and error rules as the calls above.
 */

typedef struct mi_norm_variant_info {
    int op;               /* mi_norm_op */
    int dtype;            /* mi_norm_dtype of the rows */
    int vec;              /* elements per lane access: 16 bytes' worth (4 float32,
                             8 of a 16-bit type) or 1 */
    int peel;             /* 1: per-row scalar head/tail around an aligned vector body */
    int looped;           /* 1: row streamed in chunks (re-read), any width */
    int lanes_per_row;    /* 16, 32 or 64 lanes of one wave share a row (held variants) */
    int waves_per_row;    /* waves cooperating on one row */
    int slots;            /* accesses held per lane (held variants) */
    int waves_per_block;  /* wave64s per workgroup */
    int rows_per_block;   /* rows owned by one workgroup per iteration */
    int64_t max_d;        /* widest row the variant accepts (INT64_MAX if unbounded) */
    int needs_aligned;    /* 1: 16-byte-aligned rows and parameters, strides and d
                             multiples of vec, required */
    int rows_per_lane;    /* rows whose elements a lane holds at once: 1, or 2 for
                             the multi-row variants, whose wave groups hold two rows
                             and fetch the parameters once for both */
} mi_norm_variant_info;

/* Number of compiled variants; ids are 0 .. count-1. */
int mi_norm_variant_count(void);

/* Name of variant `id`, or NULL when out of range. */
const char *mi_norm_variant_name(int id);

/* Fill *out for variant `id`.  Returns MI_NORM_ERR_INVALID when out of range. */
mi_norm_status mi_norm_variant_get_info(int id, mi_norm_variant_info *out);

/* The variant the dispatcher would choose for problem *p (host logic only,
 * no device access; eps, mean and rstd are not consulted): the storage type,
 * row width, alignment and strides pick the shape; the row count picks the
 * waves per row and the workgroup size; many rows (or rows far apart) pick a
 * multi-row variant (rows_per_lane 2).  Returns -1 when the problem's shape
 * or pointers are invalid. */
int mi_norm_select(const mi_norm_problem *p);

/* Whether variant `id` can run problem *p (1) or not (0). */
int mi_norm_eligible(int id, const mi_norm_problem *p);

/* mi_norm_fwd forced onto variant `id`.  MI_NORM_ERR_INVALID when the variant
 * does not exist, belongs to another operation or storage type, or cannot run
 * these arguments (see mi_norm_eligible). */
mi_norm_status mi_norm_fwd_variant(int id, const mi_norm_problem *p, hipStream_t stream);

/* The backward's variant queries: the variant mi_norm_bwd would run (-1 when
 * *p's shape or pointers are invalid), whether variant `id` (op
 * MI_NORM_OP_*_BWD) can run *p, and *p forced onto it. */
int mi_norm_bwd_select(const mi_norm_bwd_problem *p);
int mi_norm_bwd_eligible(int id, const mi_norm_bwd_problem *p);
mi_norm_status mi_norm_bwd_variant(int id, const mi_norm_bwd_problem *p, hipStream_t stream);

/* The named float32 calls forced onto variant `id`, as mi_norm_fwd_variant. */
mi_norm_status mi_layernorm_fwd_variant(int id, const float *x, const float *gamma,
                                        const float *beta, float *y, int64_t rows,
                                        int64_t d, float eps, float *mean, float *rstd,
                                        hipStream_t stream);
mi_norm_status mi_rmsnorm_fwd_variant(int id, const float *x, const float *w, float *y,
                                      int64_t rows, int64_t d, float eps, float *rstd,
                                      hipStream_t stream);
mi_norm_status mi_add_layernorm_fwd_variant(int id, const float *x, const float *r,
                                            const float *gamma, const float *beta, float *y,
                                            float *h, int64_t rows, int64_t d, float eps,
                                            float *mean, float *rstd, hipStream_t stream);
mi_norm_status mi_add_rmsnorm_fwd_variant(int id, const float *x, const float *r, const float *w,
                                          float *y, float *h, int64_t rows, int64_t d, float eps,
                                          float *rstd, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Calibration.  dst[i] = src[i] for i < n: a plain streaming copy with the
 * same bytes per element as the normalizations (one float32 read, one
 * written).  Benchmarks time it as the achievable-bandwidth ceiling and use it
 * to scale hardware byte counters.  src and dst must not overlap; n >= 0.
 */
mi_norm_status mi_copy_f32(const float *src, float *dst, int64_t n, hipStream_t stream);

/* The parts of a launch, for the same purpose.  kind 0: one launch of an
 * empty kernel over 256 workgroups of 1024 threads (src, dst, n unused);
 * kind 1: read n float32 from src with 16-byte non-temporal loads (nothing
 * written); kind 2: write n float32 (all 1.0f) to dst with 16-byte
 * non-temporal stores.  For kinds 1 and 2 the array is 16-byte aligned,
 * n > 0 and n % 4 == 0; MI_NORM_ERR_INVALID otherwise. */
mi_norm_status mi_calib_launch(int kind, const float *src, float *dst, int64_t n, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MI_NORM_TUNING_H */
