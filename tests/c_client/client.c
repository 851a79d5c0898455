/* A C99 caller of libmi_norm.so through its headers alone: the operations of
 * include/mi_norm.h, and the variant queries of include/mi_norm_tuning.h.
 *
 *   client layout            struct sizes and member offsets, one per line
 *   client host              results of the host-only calls (no device use)
 *   client run IN OUT R D    LayerNorm (named call, with mean/rstd) and fused
 *                            add + RMSNorm in bfloat16 (general call) of the
 *                            R x D inputs in IN; outputs written to OUT
 *
 * IN holds, as raw little-endian arrays: x float32 [R*D], gamma float32 [D],
 * beta float32 [D], then xb, rb bfloat16 bit patterns [R*D] each.  OUT holds
 * y float32 [R*D], mean [R], rstd [R], then yb, hb bfloat16 [R*D] and
 * rstdb float32 [R].  Exit status 0 on success. */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "mi_norm.h"
#include "mi_norm_tuning.h"

#define FIELD(T, m) printf("%s.%s %zu\n", #T, #m, offsetof(T, m))

static int layout(void) {
    printf("mi_norm_problem %zu\n", sizeof(mi_norm_problem));
    FIELD(mi_norm_problem, op); FIELD(mi_norm_problem, dtype); FIELD(mi_norm_problem, rows);
    FIELD(mi_norm_problem, d); FIELD(mi_norm_problem, x); FIELD(mi_norm_problem, ldx);
    FIELD(mi_norm_problem, r); FIELD(mi_norm_problem, ldr); FIELD(mi_norm_problem, y);
    FIELD(mi_norm_problem, ldy); FIELD(mi_norm_problem, h); FIELD(mi_norm_problem, ldh);
    FIELD(mi_norm_problem, params0); FIELD(mi_norm_problem, params1); FIELD(mi_norm_problem, eps);
    FIELD(mi_norm_problem, mean); FIELD(mi_norm_problem, rstd);
    printf("mi_norm_bwd_problem %zu\n", sizeof(mi_norm_bwd_problem));
    FIELD(mi_norm_bwd_problem, op); FIELD(mi_norm_bwd_problem, dtype); FIELD(mi_norm_bwd_problem, rows);
    FIELD(mi_norm_bwd_problem, d); FIELD(mi_norm_bwd_problem, dy); FIELD(mi_norm_bwd_problem, lddy);
    FIELD(mi_norm_bwd_problem, x); FIELD(mi_norm_bwd_problem, ldx); FIELD(mi_norm_bwd_problem, dx);
    FIELD(mi_norm_bwd_problem, lddx); FIELD(mi_norm_bwd_problem, params0); FIELD(mi_norm_bwd_problem, mean);
    FIELD(mi_norm_bwd_problem, rstd); FIELD(mi_norm_bwd_problem, dparams0);
    FIELD(mi_norm_bwd_problem, dparams1); FIELD(mi_norm_bwd_problem, workspace);
    FIELD(mi_norm_bwd_problem, workspace_bytes);
    printf("mi_norm_variant_info %zu\n", sizeof(mi_norm_variant_info));
    FIELD(mi_norm_variant_info, op); FIELD(mi_norm_variant_info, dtype); FIELD(mi_norm_variant_info, vec);
    FIELD(mi_norm_variant_info, peel); FIELD(mi_norm_variant_info, looped);
    FIELD(mi_norm_variant_info, lanes_per_row); FIELD(mi_norm_variant_info, waves_per_row);
    FIELD(mi_norm_variant_info, slots); FIELD(mi_norm_variant_info, waves_per_block);
    FIELD(mi_norm_variant_info, rows_per_block); FIELD(mi_norm_variant_info, max_d);
    FIELD(mi_norm_variant_info, needs_aligned); FIELD(mi_norm_variant_info, rows_per_lane);
    return 0;
}

/* addresses that are never dereferenced: the host-only calls only look at them */
#define FAKE(n) ((void *)(uintptr_t)((uint64_t)(n) << 36))

static int host(void) {
    printf("version %s\n", mi_norm_version());
    mi_norm_problem p;
    memset(&p, 0, sizeof p);
    p.op = MI_NORM_OP_LAYERNORM; p.dtype = MI_NORM_F32; p.rows = 4096; p.d = 768;
    p.x = FAKE(1); p.y = FAKE(2); p.params0 = FAKE(3); p.params1 = FAKE(4); p.eps = 1e-5f;
    printf("check_ln %d\n", (int)mi_norm_check(&p));
    int id = mi_norm_select(&p);
    printf("select_ln %s\n", id >= 0 ? mi_norm_variant_name(id) : "none");
    mi_norm_variant_info v;
    const int st = (int)mi_norm_variant_get_info(id, &v);
    printf("info_ln %d %d %d %d %d\n", st, v.waves_per_row, v.slots, v.waves_per_block, v.rows_per_lane);
    p.rows = 32768; p.d = 8192;
    id = mi_norm_select(&p);
    printf("select_big %s\n", id >= 0 ? mi_norm_variant_name(id) : "none");
    p.y = FAKE(1); p.ldy = 8000; /* y over x at another stride: rejected before any launch */
    printf("check_bad %d\n", (int)mi_norm_check(&p));
    printf("status %s\n", mi_norm_status_string(MI_NORM_ERR_INVALID));
    mi_norm_bwd_problem b;
    memset(&b, 0, sizeof b);
    b.op = MI_NORM_OP_LAYERNORM; b.dtype = MI_NORM_F32; b.rows = 4096; b.d = 768;
    b.dy = FAKE(5); b.x = FAKE(6); b.dx = FAKE(7); b.params0 = FAKE(8); b.mean = FAKE(9);
    b.rstd = FAKE(10); b.dparams0 = FAKE(11); b.dparams1 = FAKE(12);
    printf("bwd_workspace %lld\n", (long long)mi_norm_bwd_workspace_size(&b));
    printf("variants %d\n", mi_norm_variant_count());
    return 0;
}

#define HIPCHECK(call)                                                             \
    do {                                                                           \
        hipError_t e_ = (call);                                                    \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));      \
            return 3;                                                              \
        }                                                                          \
    } while (0)

#define NORMCHECK(call)                                                            \
    do {                                                                           \
        mi_norm_status s_ = (call);                                                \
        if (s_ != MI_NORM_OK) {                                                    \
            fprintf(stderr, "%s: %s\n", #call, mi_norm_status_string(s_));         \
            return 4;                                                              \
        }                                                                          \
    } while (0)

static int run(const char *in_path, const char *out_path, int64_t rows, int64_t d) {
    const size_t n = (size_t)(rows * d);
    const size_t in_bytes = 4 * n + 8 * (size_t)d + 4 * n;  /* x, gamma, beta, xb, rb */
    const size_t out_bytes = 4 * n + 8 * (size_t)rows + 4 * n + 4 * (size_t)rows;
    unsigned char *in = malloc(in_bytes), *out = malloc(out_bytes);
    if (!in || !out) return 2;
    FILE *f = fopen(in_path, "rb");
    if (!f || fread(in, 1, in_bytes, f) != in_bytes) return 2;
    fclose(f);

    void *dx, *dg, *db, *dy, *dm, *dr, *dxb, *drb, *dyb, *dhb, *drs;
    HIPCHECK(hipMalloc(&dx, 4 * n));
    HIPCHECK(hipMalloc(&dg, 4 * (size_t)d));
    HIPCHECK(hipMalloc(&db, 4 * (size_t)d));
    HIPCHECK(hipMalloc(&dy, 4 * n));
    HIPCHECK(hipMalloc(&dm, 4 * (size_t)rows));
    HIPCHECK(hipMalloc(&dr, 4 * (size_t)rows));
    HIPCHECK(hipMalloc(&dxb, 2 * n));
    HIPCHECK(hipMalloc(&drb, 2 * n));
    HIPCHECK(hipMalloc(&dyb, 2 * n));
    HIPCHECK(hipMalloc(&dhb, 2 * n));
    HIPCHECK(hipMalloc(&drs, 4 * (size_t)rows));
    const unsigned char *src = in;
    HIPCHECK(hipMemcpy(dx, src, 4 * n, hipMemcpyHostToDevice)); src += 4 * n;
    HIPCHECK(hipMemcpy(dg, src, 4 * (size_t)d, hipMemcpyHostToDevice)); src += 4 * (size_t)d;
    HIPCHECK(hipMemcpy(db, src, 4 * (size_t)d, hipMemcpyHostToDevice)); src += 4 * (size_t)d;
    HIPCHECK(hipMemcpy(dxb, src, 2 * n, hipMemcpyHostToDevice)); src += 2 * n;
    HIPCHECK(hipMemcpy(drb, src, 2 * n, hipMemcpyHostToDevice));

    /* the named float32 call, on the null stream */
    NORMCHECK(mi_layernorm_fwd(dx, dg, db, dy, rows, d, 1e-5f, dm, dr, NULL));

    /* the general call: fused add + RMSNorm over bfloat16 rows on a stream of our own */
    hipStream_t stream;
    HIPCHECK(hipStreamCreate(&stream));
    mi_norm_problem p;
    memset(&p, 0, sizeof p);
    p.op = MI_NORM_OP_ADD_RMSNORM; p.dtype = MI_NORM_BF16; p.rows = rows; p.d = d;
    p.x = dxb; p.r = drb; p.y = dyb; p.h = dhb; p.params0 = dg; p.eps = 1e-5f; p.rstd = drs;
    NORMCHECK(mi_norm_fwd(&p, stream));
    HIPCHECK(hipStreamSynchronize(stream));
    HIPCHECK(hipStreamDestroy(stream));
    HIPCHECK(hipDeviceSynchronize());

    unsigned char *dst = out;
    HIPCHECK(hipMemcpy(dst, dy, 4 * n, hipMemcpyDeviceToHost)); dst += 4 * n;
    HIPCHECK(hipMemcpy(dst, dm, 4 * (size_t)rows, hipMemcpyDeviceToHost)); dst += 4 * (size_t)rows;
    HIPCHECK(hipMemcpy(dst, dr, 4 * (size_t)rows, hipMemcpyDeviceToHost)); dst += 4 * (size_t)rows;
    HIPCHECK(hipMemcpy(dst, dyb, 2 * n, hipMemcpyDeviceToHost)); dst += 2 * n;
    HIPCHECK(hipMemcpy(dst, dhb, 2 * n, hipMemcpyDeviceToHost)); dst += 2 * n;
    HIPCHECK(hipMemcpy(dst, drs, 4 * (size_t)rows, hipMemcpyDeviceToHost));
    void *bufs[] = {dx, dg, db, dy, dm, dr, dxb, drb, dyb, dhb, drs};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIPCHECK(hipFree(bufs[i]));

    f = fopen(out_path, "wb");
    if (!f || fwrite(out, 1, out_bytes, f) != out_bytes) return 2;
    fclose(f);
    free(in);
    free(out);
    printf("ok\n");
    return 0;
}

int main(int argc, char **argv) {
    if (argc >= 2 && !strcmp(argv[1], "layout")) return layout();
    if (argc >= 2 && !strcmp(argv[1], "host")) return host();
    if (argc == 6 && !strcmp(argv[1], "run")) return run(argv[2], argv[3], atoll(argv[4]), atoll(argv[5]));
    fprintf(stderr, "usage: client layout | host | run IN OUT ROWS D\n");
    return 1;
}
