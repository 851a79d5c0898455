// mi_norm.hip — libmi_norm.so: variant table, dispatch, validation and the
// C ABI declared in include/mi_norm.h.
//
// Width dispatch mirrors the role the pages give it (mage issue #54,
// "LayerNorm [4096,768] is about 10% behind Triton's kernel": the row kernel
// covered widths up to a cap, a pair kernel the next range, and wide rows fell
// back; the fallback cost 41% at 4096 until the cap was raised).  Here every
// width has a held-row variant up to 32768 elements (128-bit path), beyond
// which a streamed-row kernel takes over, and widths that are not a multiple
// of four keep 128-bit access through a per-row peel instead of a scalar
// fallback ("Rewriting the layer norm and matmul kernels": the scalar kernel
// stayed for those widths).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstring>

#include "mi_norm.h"
#include "norm_kernels.hpp"

using namespace minorm;

namespace {

struct Variant {
    const char *name;
    mi_norm_variant_info info;
    const void *fn;
};

constexpr int64_t kUnbounded = INT64_MAX;

// Every held variant streams x in and y out with non-temporal hints and
// reads gamma/beta in the output pass (see norm_held's NTL/NTS/PRE).
#define MI_HELD(OP, OPN, VEC, PEEL, LPR, WPR, Q, WAVES)                                        \
    Variant{OPN "_" #VEC "_p" #PEEL "_l" #LPR "_w" #WPR "_q" #Q "_b" #WAVES,                  \
            mi_norm_variant_info{OP, VEC, PEEL, 0, LPR, WPR, Q, WAVES,                          \
                                 (WPR == 1) ? WAVES * (64 / LPR) : WAVES / WPR,                 \
                                 (int64_t)VEC * LPR * WPR * Q, (VEC == 4 && !PEEL) ? 1 : 0},    \
            reinterpret_cast<const void *>(                                                     \
                &norm_held<OP, VEC, (PEEL != 0), LPR, WPR, Q, WAVES, true, true, 0>)}

// the same shape with 4 and with 16 waves per workgroup
#define MI_HELD2(OP, OPN, VEC, PEEL, LPR, WPR, Q, WSMALL)                                      \
    MI_HELD(OP, OPN, VEC, PEEL, LPR, WPR, Q, WSMALL), MI_HELD(OP, OPN, VEC, PEEL, LPR, WPR, Q, 16)

#define MI_LOOP(OP, OPN, VEC, WAVES, U)                                                        \
    Variant{OPN "_" #VEC "_loop_b" #WAVES "_u" #U,                                              \
            mi_norm_variant_info{OP, VEC, 0, 1, 64, WAVES, U, WAVES, 1, kUnbounded,             \
                                 VEC == 4 ? 1 : 0},                                             \
            reinterpret_cast<const void *>(&norm_looped<OP, VEC, WAVES, U>)}

// every (waves per row, slots) pair of a 128-bit path: slots 1, 2, 3, 4, 6, 8
// for 1, 2, 4, 8 and 16 waves per row
#define MI_SLOTS(OP, OPN, PEEL, WPR, WSMALL)                                                   \
    MI_HELD2(OP, OPN, 4, PEEL, 64, WPR, 1, WSMALL), MI_HELD2(OP, OPN, 4, PEEL, 64, WPR, 2, WSMALL), \
    MI_HELD2(OP, OPN, 4, PEEL, 64, WPR, 3, WSMALL), MI_HELD2(OP, OPN, 4, PEEL, 64, WPR, 4, WSMALL), \
    MI_HELD2(OP, OPN, 4, PEEL, 64, WPR, 6, WSMALL), MI_HELD2(OP, OPN, 4, PEEL, 64, WPR, 8, WSMALL)
#define MI_SLOTS16(OP, OPN, PEEL)                                                              \
    MI_HELD(OP, OPN, 4, PEEL, 64, 16, 1, 16), MI_HELD(OP, OPN, 4, PEEL, 64, 16, 2, 16),         \
    MI_HELD(OP, OPN, 4, PEEL, 64, 16, 3, 16), MI_HELD(OP, OPN, 4, PEEL, 64, 16, 4, 16),         \
    MI_HELD(OP, OPN, 4, PEEL, 64, 16, 6, 16), MI_HELD(OP, OPN, 4, PEEL, 64, 16, 8, 16)
#define MI_PATH128(OP, OPN, PEEL)                                                              \
    MI_SLOTS(OP, OPN, PEEL, 1, 4), MI_SLOTS(OP, OPN, PEEL, 2, 4), MI_SLOTS(OP, OPN, PEEL, 4, 4), \
    MI_SLOTS(OP, OPN, PEEL, 8, 8), MI_SLOTS16(OP, OPN, PEEL)

#define MI_OP_TABLE(OP, OPN)                                                                   \
    /* 128-bit, aligned, d % 4 == 0; 16 or 32 lanes per row for narrow rows */                  \
    MI_HELD2(OP, OPN, 4, 0, 16, 1, 1, 4), MI_HELD2(OP, OPN, 4, 0, 32, 1, 1, 4),                 \
    MI_PATH128(OP, OPN, 0),                                                                     \
    /* 128-bit body with a per-row scalar head and tail: any d, x == y mod 16 B */              \
    MI_PATH128(OP, OPN, 1),                                                                     \
    /* 32-bit accesses: any d, any 4-byte alignment */                                          \
    MI_HELD2(OP, OPN, 1, 0, 16, 1, 1, 4), MI_HELD2(OP, OPN, 1, 0, 32, 1, 1, 4),                 \
    MI_HELD2(OP, OPN, 1, 0, 64, 1, 1, 4), MI_HELD2(OP, OPN, 1, 0, 64, 1, 2, 4),                 \
    MI_HELD2(OP, OPN, 1, 0, 64, 1, 4, 4), MI_HELD2(OP, OPN, 1, 0, 64, 1, 8, 4),                 \
    MI_HELD2(OP, OPN, 1, 0, 64, 4, 4, 4), MI_HELD2(OP, OPN, 1, 0, 64, 4, 8, 4),                 \
    MI_HELD2(OP, OPN, 1, 0, 64, 8, 8, 8),                                                       \
    MI_HELD(OP, OPN, 1, 0, 64, 16, 8, 16), MI_HELD(OP, OPN, 1, 0, 64, 16, 16, 16),              \
    /* streamed rows, any width */                                                             \
    MI_LOOP(OP, OPN, 4, 4, 4), MI_LOOP(OP, OPN, 1, 4, 8)

const Variant kVariants[] = {
    MI_OP_TABLE(OP_LN, "ln"),
    MI_OP_TABLE(OP_RMS, "rms"),
};
constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));

// grid cap of the grid-stride (streamed-row and copy) kernels
constexpr int64_t kMaxGrid = 1 << 20;
// row groups per launch of a held-row kernel
constexpr int64_t kMaxRowGroups = int64_t(1) << 30;

inline bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool al4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Fewest workgroups that still cover every CU: of the variants with this
// shape, the one with the most waves per workgroup whose grid has at least
// min_blocks(wpr) workgroups; failing that, the one with the most
// workgroups.  Rows of one wave need one workgroup per CU (256); rows of
// several waves share one barrier per workgroup, and 16-wave workgroups only
// paid off with two of them per CU (512).
int64_t min_blocks(int wpr) { return wpr > 1 ? 512 : 256; }

int find(int op, int64_t rows, int vec, int peel, int looped, int lpr, int wpr, int q) {
    int best = -1, fallback = -1;
    int64_t fallback_blocks = -1;
    for (int i = 0; i < kNumVariants; ++i) {
        const mi_norm_variant_info &v = kVariants[i].info;
        if (v.op != op || v.vec != vec || v.peel != peel || v.looped != looped) continue;
        if (looped) return i;
        if (v.lanes_per_row != lpr || v.waves_per_row != wpr || v.slots != q) continue;
        const int64_t blocks = (rows + v.rows_per_block - 1) / v.rows_per_block;
        if (blocks >= min_blocks(wpr) && (best < 0 || v.waves_per_block > kVariants[best].info.waves_per_block))
            best = i;
        if (blocks > fallback_blocks) {
            fallback = i;
            fallback_blocks = blocks;
        }
    }
    return best >= 0 ? best : fallback;
}

// smallest listed slot count q with cap_per_slot * q >= n, or 0
int pick_q(int64_t n, int64_t cap_per_slot, const int *qs, int nq) {
    for (int i = 0; i < nq; ++i)
        if (cap_per_slot * qs[i] >= n) return qs[i];
    return 0;
}

// Waves per row and slots for a 128-bit row of nvec accesses (wpr = 0 when
// the row is too wide to hold).  About four 16-byte accesses per lane
// measured best across widths (more per lane cut occupancy, fewer add
// waves and exchange traffic); with few rows, a row is spread over more waves
// until the grid holds 4096 waves, as long as every wave keeps one full
// access per lane.
void shape128(int64_t nvec, int64_t rows, int &wpr, int &q) {
    static const int qs[] = {1, 2, 3, 4, 6, 8};
    wpr = 1;
    while (wpr < 16 && 64 * wpr * 4 < nvec) wpr *= 2;
    while (wpr < 16 && rows * wpr < 4096 && nvec >= 64 * 2 * wpr) wpr *= 2;
    q = pick_q(nvec, 64 * wpr, qs, 6);
    if (q == 0) wpr = 0;
}

void ladder1(int64_t n, int &lpr, int &wpr, int &q) {
    static const int q1[] = {1, 2, 4, 8};
    static const int q4[] = {4, 8};
    static const int q16[] = {8, 16};
    lpr = 64;
    wpr = 0;
    q = 0;
    if (n <= 16) { lpr = 16; wpr = 1; q = 1; return; }
    if (n <= 32) { lpr = 32; wpr = 1; q = 1; return; }
    if (n <= 512) { wpr = 1; q = pick_q(n, 64, q1, 4); return; }
    if (n <= 2048) { wpr = 4; q = pick_q(n, 256, q4, 2); return; }
    if (n <= 4096) { wpr = 8; q = 8; return; }
    if (n <= 16384) { wpr = 16; q = pick_q(n, 1024, q16, 2); return; }
}

struct Layout {
    bool a16;      // every pointer 16-byte aligned and d % 4 == 0
    bool peel_ok;  // x and y share their phase within 16 bytes
};

Layout layout_of(int op, int64_t d, const void *x, const void *y, const void *p0, const void *p1) {
    Layout L;
    L.a16 = (d % 4 == 0) && al16(x) && al16(y) && al16(p0) && (op == OP_RMS || al16(p1));
    L.peel_ok = ((reinterpret_cast<uintptr_t>(x) ^ reinterpret_cast<uintptr_t>(y)) & 15u) == 0;
    return L;
}

bool args_ok(int op, int64_t d, const void *x, const void *y, const void *p0, const void *p1) {
    if (op != OP_LN && op != OP_RMS) return false;
    if (!x || !y || !p0 || (op == OP_LN && !p1)) return false;
    if (!al4(x) || !al4(y) || !al4(p0) || (op == OP_LN && !al4(p1))) return false;
    if (d < 1 || d > INT32_MAX) return false;
    return true;
}

int select_variant(int op, int64_t rows, int64_t d, const void *x, const void *y, const void *p0,
                   const void *p1) {
    if (!args_ok(op, d, x, y, p0, p1) || rows < 0) return -1;
    const Layout L = layout_of(op, d, x, y, p0, p1);
    int lpr, wpr, q;
    if (L.a16) {
        const int64_t nvec = d / 4;
        if (nvec <= 16) return find(op, rows, 4, 0, 0, 16, 1, 1);
        if (nvec <= 32) return find(op, rows, 4, 0, 0, 32, 1, 1);
        shape128(nvec, rows, wpr, q);
        if (wpr) return find(op, rows, 4, 0, 0, 64, wpr, q);
        return find(op, rows, 4, 0, 1, 0, 0, 0);
    }
    if (L.peel_ok && d >= 256) {
        shape128((d + 3) / 4, rows, wpr, q);
        if (wpr) return find(op, rows, 4, 1, 0, 64, wpr, q);
        return find(op, rows, 1, 0, 1, 0, 0, 0);
    }
    ladder1(d, lpr, wpr, q);
    if (wpr) return find(op, rows, 1, 0, 0, lpr, wpr, q);
    return find(op, rows, 1, 0, 1, 0, 0, 0);
}

bool eligible(int id, int op, int64_t d, const void *x, const void *y, const void *p0, const void *p1) {
    if (id < 0 || id >= kNumVariants) return false;
    if (!args_ok(op, d, x, y, p0, p1)) return false;
    const mi_norm_variant_info &v = kVariants[id].info;
    if (v.op != op) return false;
    const Layout L = layout_of(op, d, x, y, p0, p1);
    if (v.looped) return v.vec == 1 || L.a16;
    if (v.peel) return L.peel_ok && (d + 3) / 4 <= v.max_d / 4;
    if (v.vec == 4) return L.a16 && d <= v.max_d;
    return d <= v.max_d;
}

// y may equal x; otherwise the two [rows, d] ranges must not intersect
bool overlap_ok(const void *x, const void *y, int64_t rows, int64_t d) {
    if (x == y || rows == 0) return true;
    const uintptr_t bytes = (uintptr_t)rows * (uintptr_t)d * sizeof(float);
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
    return a + bytes <= b || b + bytes <= a;
}

// [a, a + na) and [b, b + nb) (in floats) intersect
bool ranges_meet(const void *a, int64_t na, const void *b, int64_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + (uintptr_t)nb * sizeof(float) && pb < pa + (uintptr_t)na * sizeof(float);
}

mi_norm_status validate(int op, const float *x, const float *p0, const float *p1, const float *y,
                        int64_t rows, int64_t d, float eps, const float *mean, const float *rstd) {
    if (!args_ok(op, d, x, y, p0, p1)) return MI_NORM_ERR_INVALID;
    if (rows < 0) return MI_NORM_ERR_INVALID;
    if (!(eps >= 0.f)) return MI_NORM_ERR_INVALID;  // also rejects NaN
    if (rows > 0 && rows > (INT64_MAX / (int64_t)sizeof(float)) / d) return MI_NORM_ERR_INVALID;
    if ((mean && !al4(mean)) || (rstd && !al4(rstd))) return MI_NORM_ERR_INVALID;
    if (!overlap_ok(x, y, rows, d)) return MI_NORM_ERR_INVALID;
    // parameters are read after earlier slots of y are stored
    if (rows > 0 && (ranges_meet(y, rows * d, p0, d) || (p1 && ranges_meet(y, rows * d, p1, d))))
        return MI_NORM_ERR_INVALID;
    return MI_NORM_OK;
}

// Held variants give each workgroup one row group, so the grid is
// ceil(rows / rows_per_block).  Only a row count beyond kMaxRowGroups row
// groups (2^30, far past device memory for any width) is split over several
// launches; streamed variants walk rows with a grid-stride loop.
mi_norm_status launch(int id, const NormParams &P, hipStream_t stream) {
    if (P.rows == 0) return MI_NORM_OK;
    const Variant &v = kVariants[id];
    const dim3 block(v.info.waves_per_block * 64);
    if (v.info.looped) {
        const int64_t blocks = P.rows < kMaxGrid ? P.rows : kMaxGrid;
        NormParams arg = P;
        void *args[] = {&arg};
        return hipLaunchKernel(v.fn, dim3((unsigned)blocks), block, args, 0, stream) == hipSuccess
                   ? MI_NORM_OK : MI_NORM_ERR_HIP;
    }
    const int64_t rpb = v.info.rows_per_block;
    const int64_t chunk = kMaxRowGroups * rpb;
    for (int64_t r0 = 0; r0 < P.rows; r0 += chunk) {
        NormParams arg = P;
        const int64_t n = (P.rows - r0) < chunk ? (P.rows - r0) : chunk;
        arg.rows = n;
        arg.x = P.x + r0 * (int64_t)P.d;
        arg.y = P.y + r0 * (int64_t)P.d;
        if (P.mean) arg.mean = P.mean + r0;
        if (P.rstd) arg.rstd = P.rstd + r0;
        void *args[] = {&arg};
        const int64_t blocks = (n + rpb - 1) / rpb;
        if (hipLaunchKernel(v.fn, dim3((unsigned)blocks), block, args, 0, stream) != hipSuccess)
            return MI_NORM_ERR_HIP;
    }
    return MI_NORM_OK;
}

NormParams make_params(const float *x, const float *p0, const float *p1, float *y, int64_t rows,
                       int64_t d, float eps, float *mean, float *rstd) {
    NormParams P;
    P.x = x;
    P.p0 = p0;
    P.p1 = p1;
    P.y = y;
    P.mean = mean;
    P.rstd = rstd;
    P.rows = rows;
    P.d = (int32_t)d;
    P.eps = eps;
    P.inv_d = (float)(1.0 / (double)d);
    return P;
}

mi_norm_status run(int op, int forced, const float *x, const float *p0, const float *p1, float *y,
                   int64_t rows, int64_t d, float eps, float *mean, float *rstd, hipStream_t stream) {
    const mi_norm_status st = validate(op, x, p0, p1, y, rows, d, eps, mean, rstd);
    if (st != MI_NORM_OK) return st;
    int id = forced;
    if (id < 0) {
        id = select_variant(op, rows, d, x, y, p0, p1);
        if (id < 0) return MI_NORM_ERR_INVALID;
    } else if (!eligible(id, op, d, x, y, p0, p1)) {
        return MI_NORM_ERR_INVALID;
    }
    if (rows == 0) return MI_NORM_OK;
    return launch(id, make_params(x, p0, p1, y, rows, d, eps, mean, rstd), stream);
}

}  // namespace

extern "C" {

const char *mi_norm_status_string(mi_norm_status s) {
    switch (s) {
    case MI_NORM_OK: return "MI_NORM_OK";
    case MI_NORM_ERR_INVALID: return "MI_NORM_ERR_INVALID: invalid argument, nothing launched";
    case MI_NORM_ERR_HIP: return "MI_NORM_ERR_HIP: kernel launch failed";
    }
    return "MI_NORM_UNKNOWN_STATUS";
}

const char *mi_norm_version(void) { return "mi_norm 0.1.0 gfx950"; }

mi_norm_status mi_layernorm_fwd(const float *x, const float *gamma, const float *beta, float *y,
                                int64_t rows, int64_t d, float eps, float *mean, float *rstd,
                                hipStream_t stream) {
    return run(OP_LN, -1, x, gamma, beta, y, rows, d, eps, mean, rstd, stream);
}

mi_norm_status mi_rmsnorm_fwd(const float *x, const float *w, float *y, int64_t rows, int64_t d,
                              float eps, float *rstd, hipStream_t stream) {
    return run(OP_RMS, -1, x, w, nullptr, y, rows, d, eps, nullptr, rstd, stream);
}

int mi_norm_variant_count(void) { return kNumVariants; }

const char *mi_norm_variant_name(int id) {
    return (id >= 0 && id < kNumVariants) ? kVariants[id].name : nullptr;
}

mi_norm_status mi_norm_variant_get_info(int id, mi_norm_variant_info *out) {
    if (id < 0 || id >= kNumVariants || !out) return MI_NORM_ERR_INVALID;
    *out = kVariants[id].info;
    return MI_NORM_OK;
}

int mi_norm_select_variant(int op, int64_t rows, int64_t d, const void *x, const void *y,
                           const void *params0, const void *params1) {
    return select_variant(op, rows, d, x, y, params0, params1);
}

int mi_norm_variant_eligible(int id, int op, int64_t d, const void *x, const void *y,
                             const void *params0, const void *params1) {
    return eligible(id, op, d, x, y, params0, params1) ? 1 : 0;
}

mi_norm_status mi_layernorm_fwd_variant(int id, const float *x, const float *gamma, const float *beta,
                                        float *y, int64_t rows, int64_t d, float eps, float *mean,
                                        float *rstd, hipStream_t stream) {
    if (id < 0 || id >= kNumVariants) return MI_NORM_ERR_INVALID;
    return run(OP_LN, id, x, gamma, beta, y, rows, d, eps, mean, rstd, stream);
}

mi_norm_status mi_rmsnorm_fwd_variant(int id, const float *x, const float *w, float *y, int64_t rows,
                                      int64_t d, float eps, float *rstd, hipStream_t stream) {
    if (id < 0 || id >= kNumVariants) return MI_NORM_ERR_INVALID;
    return run(OP_RMS, id, x, w, nullptr, y, rows, d, eps, nullptr, rstd, stream);
}

mi_norm_status mi_copy_f32(const float *src, float *dst, int64_t n, hipStream_t stream) {
    if (n < 0) return MI_NORM_ERR_INVALID;
    if (n == 0) return MI_NORM_OK;
    if (!src || !dst || !al4(src) || !al4(dst)) return MI_NORM_ERR_INVALID;
    if (n > INT64_MAX / (int64_t)sizeof(float)) return MI_NORM_ERR_INVALID;
    if (!overlap_ok(src, dst, 1, n) || src == dst) return MI_NORM_ERR_INVALID;
    hipError_t e;
    if (n % 4 == 0 && al16(src) && al16(dst)) {
        // one 128-bit access per lane for large copies, two below 256 MiB
        // (the faster shapes on gfx950 at 2 GiB and at 24 MiB)
        const int64_t n4 = n / 4;
        const bool big = n4 >= (int64_t(1) << 24);
        const int U = big ? 1 : 2;
        int64_t blocks = (n4 + 256 * U - 1) / (256 * U);
        if (blocks > kMaxGrid) blocks = kMaxGrid;
        int64_t n4a = n4;
        const float *s = src;
        float *dd = dst;
        void *args[] = {&s, &dd, &n4a};
        const void *fn = big ? reinterpret_cast<const void *>(&copy_f4<1>)
                             : reinterpret_cast<const void *>(&copy_f4<2>);
        e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0, stream);
    } else {
        int64_t blocks = (n + 255) / 256;
        if (blocks > kMaxGrid) blocks = kMaxGrid;
        int64_t na = n;
        const float *s = src;
        float *dd = dst;
        void *args[] = {&s, &dd, &na};
        e = hipLaunchKernel(reinterpret_cast<const void *>(&copy_f1), dim3((unsigned)blocks), dim3(256),
                            args, 0, stream);
    }
    return e == hipSuccess ? MI_NORM_OK : MI_NORM_ERR_HIP;
}

}  // extern "C"
