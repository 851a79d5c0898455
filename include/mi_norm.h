/*
 * mi_norm.h — C ABI of libmi_norm.so: forward row-wise normalization of a
 * [rows, d] matrix (float32, binary16 or bfloat16 rows, any row stride) on
 * AMD Instinct MI355X (gfx950).
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
 * Residual add fused before either norm (the RMSNorm page, same section,
 * lists fusion with a residual add among what its kernels leave out):
 *     h = x + r (rounded to the row storage type, optionally written out),
 *     y = Norm(h)
 *
 * Arithmetic is IEEE float32 with fused multiply-adds and the hardware
 * reciprocal square root; results agree with a float64 evaluation of the same
 * definition within |err| <= 1e-5 + 1e-4 * |ref| (the acceptance bound of the
 * RMSNorm page, section "Correctness before timing").
 *
 * Storage types.  Rows (x, r, y, h) may be float32, IEEE binary16 or
 * bfloat16 (mi_norm_dtype).  16-bit rows are widened exactly to float32, the
 * statistics and arithmetic stay float32, parameters (gamma, beta, w) and the
 * statistics outputs (mean, rstd) are always float32, and each 16-bit output
 * is rounded once, to nearest with ties to even.  A 16-bit y is therefore
 * within the float32 bound above plus half a unit in the last place of the
 * 16-bit format; h is the storage-format rounding of x + r, exactly.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers (HIP device memory of the current device),
 *   aligned to their element size.  The row tensors x, r, y, h are row-major
 *   [rows, d]: element (i, j) at base + i * ld + j elements, where the named
 *   float32 calls use ld = d and mi_norm_fwd takes one ld per tensor
 *   (ld >= d; 0 means d).  gamma, beta and w are float32 [d]; mean and rstd
 *   are float32 [rows].
 * - Ownership: the caller allocates, owns and frees every buffer.  The library
 *   allocates, frees and synchronizes nothing, keeps no global mutable state
 *   and is reentrant; calls on different streams may run concurrently.
 * - Work is enqueued on `stream` (NULL = the null stream) and the call returns
 *   without waiting.  One kernel launch per call; calls may be captured into a
 *   HIP graph.
 * - Aliasing: an output row tensor (y, h) either IS an input row tensor
 *   (x or r: same pointer, same row stride — in place) or shares no element
 *   with any other row tensor; y and h never share an element.  Inputs may
 *   overlap each other freely (e.g. x and r interleaved in one buffer).  No
 *   output may overlap gamma, beta or w, and mean/rstd may overlap no other
 *   argument.
 * - Row tensors 16-byte aligned, with d and every row stride a multiple of
 *   the elements in 16 bytes (4 float32, 8 of a 16-bit type), and 16-byte
 *   aligned parameters select the vector path (16-byte accesses); rows that
 *   share their phase within 16 bytes take a peeled vector path; any other
 *   layout a scalar path with the same results.
 * - Errors: MI_NORM_ERR_INVALID is returned before any launch for a NULL
 *   required pointer, a misaligned pointer, an unknown op or dtype, rows < 0,
 *   d < 1, d > 2^31 - 2^16, a row stride below d, a size overflow, eps NaN or
 *   negative, or an aliasing pattern the rule above excludes.  rows == 0
 *   returns MI_NORM_OK and launches nothing.
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
 * The general call: any of the four operations over float32, binary16 or
 * bfloat16 rows with a row stride per tensor, described by one struct.
 */

typedef enum mi_norm_op {
    MI_NORM_OP_LAYERNORM = 0,
    MI_NORM_OP_RMSNORM = 1,
    MI_NORM_OP_ADD_LAYERNORM = 2,  /* residual add fused before LayerNorm */
    MI_NORM_OP_ADD_RMSNORM = 3,    /* residual add fused before RMSNorm */
    MI_NORM_OP_LAYERNORM_BWD = 4,  /* (variant table only) LayerNorm backward */
    MI_NORM_OP_RMSNORM_BWD = 5     /* (variant table only) RMSNorm backward */
} mi_norm_op;

typedef enum mi_norm_dtype {
    MI_NORM_F32 = 0,   /* IEEE binary32 */
    MI_NORM_F16 = 1,   /* IEEE binary16 */
    MI_NORM_BF16 = 2   /* bfloat16: binary32's exponent, 8 significand bits */
} mi_norm_dtype;

/* One call in full.  Row strides are in elements (0 means d). */
typedef struct mi_norm_problem {
    int op;                 /* mi_norm_op */
    int dtype;              /* mi_norm_dtype of x, r, y and h */
    int64_t rows;           /* >= 0 */
    int64_t d;              /* >= 1 */
    const void *x;          /* input rows                                      (required) */
    int64_t ldx;
    const void *r;          /* residual rows (MI_NORM_OP_ADD_*), else ignored  */
    int64_t ldr;
    void *y;                /* output rows                                     (required) */
    int64_t ldy;
    void *h;                /* x + r rows (MI_NORM_OP_ADD_*), NULL to skip     */
    int64_t ldh;
    const float *params0;   /* gamma (LayerNorm ops) or w, float32 [d]         (required) */
    const float *params1;   /* beta (LayerNorm ops, required), else ignored    */
    float eps;              /* >= 0 */
    float *mean;            /* float32 [rows] or NULL (LayerNorm ops only)     */
    float *rstd;            /* float32 [rows] or NULL                          */
} mi_norm_problem;

/* Run problem *p on `stream`: the named calls above are this call with dtype
 * MI_NORM_F32 and every row stride d.  A NULL p is MI_NORM_ERR_INVALID. */
mi_norm_status mi_norm_fwd(const mi_norm_problem *p, hipStream_t stream);

/* The argument checks of mi_norm_fwd alone (host logic, nothing launched, no
 * device access): MI_NORM_OK when mi_norm_fwd would accept *p. */
mi_norm_status mi_norm_check(const mi_norm_problem *p);

/* ---------------------------------------------------------------------------
 * Backward.  The gradients of the two normalizations with respect to the rows
 * and the parameters, from the upstream gradient dy and the per-row
 * statistics the forward returned.  They are the exact derivative of the
 * definitions above; no page defines them.  Per row i, with
 * xhat_ij = (x_ij - mean_i) * rstd_i (RMSNorm: x_ij * rstd_i) and
 * g_ij = dy_ij * gamma_j (RMSNorm: dy_ij * w_j):
 *     LayerNorm  dx_ij = rstd_i * (g_ij - mean_k g_ik - xhat_ij * mean_k(g_ik xhat_ik))
 *     RMSNorm    dx_ij = rstd_i * (g_ij - xhat_ij * mean_k(g_ik xhat_ik))
 * and over all rows dgamma_j (dw_j) = sum_i dy_ij xhat_ij, dbeta_j = sum_i dy_ij.
 *
 * dy, x and dx share a storage type (float32, binary16, bfloat16; each with
 * its own row stride); gamma/w, mean, rstd, dgamma/dw and dbeta are float32.
 * Arithmetic: every term (g, g xhat, dy xhat, dy) is formed in float32 from
 * the float32 inputs.  A row's two sums add at most eight consecutive terms
 * in float32 and carry the rest in float64; each mean is rounded once to
 * float32.  A column sum is carried in float64, rounded to float32 at most
 * twice on the way (once for a subset of a workgroup's rows, once for the
 * workgroup's), the workgroups' partial rows added in float64 in a fixed
 * order and rounded once (deterministic results).  Hence, with u = 2^-24
 * and whatever the launch shape, dx is within 1e-5 + 1e-4 |ref| +
 * 16 u rstd_i (|g_ij| + mean_k |g_ik| + |xhat_ij| mean_k |g_ik xhat_ik|) of
 * the float64 derivative (plus half a 16-bit ulp for 16-bit dx; the
 * subtraction of the row means amplifies float32 rounding by rstd, which is
 * large for rows of near-zero variance), and the parameter gradients within
 * 1e-5 + 1e-4 |ref| + 6 u sum_i |term_i|.
 *
 * The parameter gradients need device scratch memory that the caller owns:
 * mi_norm_bwd_workspace_size says how many bytes (it depends on the shape
 * only); the pointer must be 256-byte aligned.  Its contents on entry do not
 * matter and are overwritten; it must not overlap any other argument, and two
 * calls in flight at once need two workspaces.  With dparams0 and dparams1
 * both NULL only dx is computed (the workspace may still be needed for rows
 * wider than the held variants).
 *
 * Aliasing: dx may be dy or x in place (same pointer and stride) or share no
 * element with them; dgamma, dbeta and the workspace overlap nothing.  Each
 * call launches two or three kernels on `stream`.
 */
typedef struct mi_norm_bwd_problem {
    int op;                 /* MI_NORM_OP_LAYERNORM or MI_NORM_OP_RMSNORM */
    int dtype;              /* mi_norm_dtype of dy, x and dx */
    int64_t rows;           /* >= 0 */
    int64_t d;              /* >= 1 and <= 2^31 - 2^16, as for the forward */
    const void *dy;         /* upstream gradient rows                         (required) */
    int64_t lddy;
    const void *x;          /* the forward's input rows                       (required) */
    int64_t ldx;
    void *dx;               /* gradient rows out                              (required) */
    int64_t lddx;
    const float *params0;   /* gamma or w, float32 [d]                        (required) */
    const float *mean;      /* float32 [rows] from the forward (LayerNorm)    (required) */
    const float *rstd;      /* float32 [rows] from the forward                (required) */
    float *dparams0;        /* dgamma or dw, float32 [d], or NULL to skip     */
    float *dparams1;        /* dbeta, float32 [d] (LayerNorm), or NULL        */
    void *workspace;        /* device scratch, 256-byte aligned                */
    int64_t workspace_bytes;
} mi_norm_bwd_problem;

/* Bytes of workspace mi_norm_bwd needs for *p (its op, dtype, rows, d and
 * which parameter gradients are wanted; no pointer is consulted); -1 when
 * those are invalid. */
int64_t mi_norm_bwd_workspace_size(const mi_norm_bwd_problem *p);

/* Run the backward described by *p on `stream`. */
mi_norm_status mi_norm_bwd(const mi_norm_bwd_problem *p, hipStream_t stream);

/* The argument checks of mi_norm_bwd alone (nothing launched). */
mi_norm_status mi_norm_bwd_check(const mi_norm_bwd_problem *p);

/* mi_norm_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and results, with the workspace taken from a scratch array
 * the library holds on each GPU (32 MiB, held from the library's first use
 * on that GPU until the process ends) instead of the caller's.
 * p->workspace must be NULL and p->workspace_bytes 0.  Returns
 * MI_NORM_ERR_INVALID, launching nothing, when the problem needs more
 * workspace than the array holds (mi_norm_bwd_workspace_size(p) >
 * mi_norm_bwd_noalloc_limit(): LayerNorm with d up to 8192 fits for up to
 * 2 million rows) and MI_NORM_ERR_HIP when the array's address cannot be
 * had.  The stream must belong to the current device.  The call allocates
 * and frees nothing.  Every call on one GPU shares that GPU's array, whose
 * contents on entry do not matter: calls that overlap in time on one GPU
 * (different streams, or host threads) race on it and must be serialized by
 * the caller. */
mi_norm_status mi_norm_bwd_noalloc(const mi_norm_bwd_problem *p, hipStream_t stream);

/* Bytes of the scratch array mi_norm_bwd_noalloc uses (33554432). */
int64_t mi_norm_bwd_noalloc_limit(void);

/* The float32 contiguous forms (row stride d). */
mi_norm_status mi_layernorm_bwd(const float *dy, const float *x, const float *gamma,
                                const float *mean, const float *rstd, float *dx,
                                float *dgamma, float *dbeta, int64_t rows, int64_t d,
                                void *workspace, int64_t workspace_bytes, hipStream_t stream);
mi_norm_status mi_rmsnorm_bwd(const float *dy, const float *x, const float *w,
                              const float *rstd, float *dx, float *dw, int64_t rows, int64_t d,
                              void *workspace, int64_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MI_NORM_H */
