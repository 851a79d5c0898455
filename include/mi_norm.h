/*
 * mi_norm.h — C ABI of libmi_norm.so: forward row-wise normalization of a
 * contiguous float32 [rows, d] matrix on AMD Instinct MI355X (gfx950).
 *
 * Operations
 * ----------
 * LayerNorm.  Per row i the mean and the biased, centered variance are the two
 * reductions of the equation in "Rewriting the layer norm and matmul kernels"
 * (section "A reduction has to meet somewhere"):
 *     mu_i = (1/d) sum_j x_ij,   sigma_i^2 = (1/d) sum_j (x_ij - mu_i)^2
 * and the output applies the per-column scale and bias that the kernels of
 * "Field note 004: The load in flight, and the shape Triton uses" (section
 * "The layer norm was rewritten in the shape Triton uses") load beside x:
 *     y_ij = (x_ij - mu_i) * rsqrt(sigma_i^2 + eps) * gamma_j + beta_j
 *
 * RMSNorm.  As the equation of "RMSNorm on an RTX 5070: why more reduction
 * threads did not win every shape" (section "The operator and the change"):
 *     y_rc = x_rc * w_c * rsqrt((1/d) sum_j x_rj^2 + eps)
 *
 * Residual add fused before either norm (the step before the normalization
 * whose absence the RMSNorm page notes: "no ... fusion with a residual add"):
 *     h = x + r (a float32 addition, optionally written out), y = Norm(h)
 *
 * Arithmetic is IEEE float32 with fused multiply-adds and the hardware
 * reciprocal square root; results agree with a float64 evaluation of the same
 * definition within |err| <= 1e-5 + 1e-4 * |ref| (the acceptance bound of the
 * RMSNorm page, section "Correctness before timing").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers (HIP device memory of the current device),
 *   float32, 4-byte aligned.  x and y are row-major [rows, d] with row stride
 *   d; gamma, beta and w are [d]; mean and rstd are [rows].
 * - Ownership: the caller allocates, owns and frees every buffer.  The library
 *   allocates, frees and synchronizes nothing, keeps no global mutable state
 *   and is reentrant; calls on different streams may run concurrently.
 * - Work is enqueued on `stream` (NULL = the null stream) and the call returns
 *   without waiting.  One kernel launch per call; calls may be captured into a
 *   HIP graph.
 * - Aliasing: the [rows, d] tensors (x, y, and for the fused calls r, h) are
 *   each either the same pointer as another or disjoint from it: y may equal
 *   x (in place), and in the fused calls y and h may each equal x or r, but y
 *   and h never share memory.  An output overlapping gamma, beta or w is
 *   rejected.  mean/rstd must not overlap any other argument.
 * - 16-byte-aligned x, y, gamma, beta (or w) and d % 4 == 0 select the
 *   128-bit vector path; other layouts take a peeled or scalar path with the
 *   same results.
 * - Errors: MI_NORM_ERR_INVALID is returned before any launch for a NULL
 *   required pointer, a pointer not 4-byte aligned, rows < 0, d < 1,
 *   d > 2^31 - 1, a size overflow, eps NaN or negative, or an aliasing
 *   pattern the rule above excludes.  rows == 0 returns MI_NORM_OK and launches nothing.
 *   MI_NORM_ERR_HIP reports a failed launch (the HIP error is not kept;
 *   faults inside the kernel surface at the caller's next synchronization,
 *   as usual for HIP).  No C++ exception crosses this interface.
 * - Non-finite inputs are outside the contract and propagate.
 *
 * Consumers compile against HIP's headers (hipcc does this; with gcc/clang
 * pass -D__HIP_PLATFORM_AMD__ -I/opt/rocm/include).
 */
#ifndef MI_NORM_H
#define MI_NORM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mi_norm_status {
    MI_NORM_OK = 0,
    MI_NORM_ERR_INVALID = 1,  /* bad argument; nothing was launched */
    MI_NORM_ERR_HIP = 2       /* the HIP launch failed */
} mi_norm_status;

/* Human-readable name of a status code (static storage, never NULL). */
const char *mi_norm_status_string(mi_norm_status s);

/* Library version string (static storage). */
const char *mi_norm_version(void);

/*
 * LayerNorm forward.
 *   x      [rows, d]  input                         (required)
 *   gamma  [d]        per-column scale              (required)
 *   beta   [d]        per-column shift              (required)
 *   y      [rows, d]  output; may equal x           (required)
 *   rows   >= 0; d >= 1
 *   eps    >= 0, added to the variance inside the root (1e-5 is usual)
 *   mean   [rows]     per-row mean mu_i, or NULL to skip
 *   rstd   [rows]     per-row 1/sqrt(sigma_i^2 + eps), or NULL to skip
 *   stream HIP stream to enqueue on (NULL = null stream)
 */
mi_norm_status mi_layernorm_fwd(const float *x, const float *gamma, const float *beta,
                                float *y, int64_t rows, int64_t d, float eps,
                                float *mean, float *rstd, hipStream_t stream);

/*
 * RMSNorm forward.
 *   x      [rows, d]  input                         (required)
 *   w      [d]        per-column weight             (required)
 *   y      [rows, d]  output; may equal x           (required)
 *   rows   >= 0; d >= 1
 *   eps    >= 0, added to the mean square inside the root
 *   rstd   [rows]     per-row 1/sqrt(mean(x^2) + eps), or NULL to skip
 *   stream HIP stream to enqueue on (NULL = null stream)
 */
mi_norm_status mi_rmsnorm_fwd(const float *x, const float *w, float *y,
                              int64_t rows, int64_t d, float eps,
                              float *rstd, hipStream_t stream);

/*
 * Residual add + LayerNorm forward: h = x + r (float32), y = LayerNorm(h).
 *   x, r   [rows, d]  inputs                        (required)
 *   gamma, beta [d]   per-column scale and shift    (required)
 *   y      [rows, d]  output; may equal x or r      (required)
 *   h      [rows, d]  x + r; may equal x or r; never y; NULL to skip
 *   mean, rstd [rows] statistics of h, or NULL to skip
 * Other arguments as mi_layernorm_fwd.  One kernel reads x and r once and
 * writes y (and h): 12 (16) bytes per element instead of the 20 of a
 * separate add and norm.
 */
mi_norm_status mi_add_layernorm_fwd(const float *x, const float *r, const float *gamma,
                                    const float *beta, float *y, float *h,
                                    int64_t rows, int64_t d, float eps,
                                    float *mean, float *rstd, hipStream_t stream);

/* Residual add + RMSNorm forward: h = x + r (float32), y = RMSNorm(h); the
 * arguments follow mi_add_layernorm_fwd and mi_rmsnorm_fwd. */
mi_norm_status mi_add_rmsnorm_fwd(const float *x, const float *r, const float *w,
                                  float *y, float *h, int64_t rows, int64_t d, float eps,
                                  float *rstd, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Kernel variants.  Every call above is served by one compiled kernel variant
 * chosen from the operation, the row width d, the pointer alignment and the
 * row count.  The calls below expose that
 * table so tests can drive every variant and benchmarks can compare them.
 * They follow the same conventions and error rules as the calls above.
 */

typedef enum mi_norm_op {
    MI_NORM_OP_LAYERNORM = 0,
    MI_NORM_OP_RMSNORM = 1,
    MI_NORM_OP_ADD_LAYERNORM = 2,  /* residual add fused before LayerNorm */
    MI_NORM_OP_ADD_RMSNORM = 3     /* residual add fused before RMSNorm */
} mi_norm_op;

/* One call's shape and pointers, for the variant queries below. */
typedef struct mi_norm_problem {
    int op;                 /* mi_norm_op */
    int64_t rows;
    int64_t d;
    const void *x;          /* input */
    const void *r;          /* residual input (MI_NORM_OP_ADD_*), else ignored */
    const void *y;          /* output */
    const void *h;          /* x + r output (MI_NORM_OP_ADD_*), NULL if not written */
    const void *params0;    /* gamma or w */
    const void *params1;    /* beta (LayerNorm ops), else ignored */
} mi_norm_problem;

typedef struct mi_norm_variant_info {
    int op;               /* mi_norm_op */
    int vec;              /* elements per lane access: 4 (128-bit) or 1 */
    int peel;             /* 1: per-row scalar head/tail around an aligned 128-bit body */
    int looped;           /* 1: row streamed in chunks (re-read), any width */
    int lanes_per_row;    /* 16, 32 or 64 lanes of one wave share a row (held variants) */
    int waves_per_row;    /* waves cooperating on one row */
    int slots;            /* accesses held per lane (held variants) */
    int waves_per_block;  /* wave64s per workgroup */
    int rows_per_block;   /* rows owned by one workgroup per iteration */
    int64_t max_d;        /* widest row the variant accepts (INT64_MAX if unbounded) */
    int needs_aligned;    /* 1: x, y, params 16-byte aligned and d % 4 == 0 required */
} mi_norm_variant_info;

/* Number of compiled variants; ids are 0 .. count-1. */
int mi_norm_variant_count(void);

/* Name of variant `id`, or NULL when out of range. */
const char *mi_norm_variant_name(int id);

/* Fill *out for variant `id`.  Returns MI_NORM_ERR_INVALID when out of range. */
mi_norm_status mi_norm_variant_get_info(int id, mi_norm_variant_info *out);

/* The variant the dispatcher would choose for problem *p (host logic only,
 * no device access): the row width and pointer alignment pick the shape, the
 * row count picks the waves per row and the workgroup size.  Returns -1 when
 * the problem is invalid. */
int mi_norm_select(const mi_norm_problem *p);

/* Whether variant `id` can run problem *p (1) or not (0). */
int mi_norm_eligible(int id, const mi_norm_problem *p);

/* LayerNorm / RMSNorm forced onto variant `id`.  MI_NORM_ERR_INVALID when the
 * variant does not exist, belongs to the other operation, or cannot run these
 * arguments (see mi_norm_variant_eligible). */
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

#ifdef __cplusplus
}
#endif

#endif /* MI_NORM_H */
