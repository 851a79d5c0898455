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

// ABI op codes: bit 0 picks the normalization, op >= 2 fuses the residual add
constexpr int kOps = 4;
constexpr int kop(int op) { return op & 1; }       // OP_LN or OP_RMS
constexpr bool kres(int op) { return op >= 2; }

// Every held variant streams x (and r) in and y (and h) out with
// non-temporal hints and reads gamma/beta in the output pass (norm_held's
// NTL/NTS/PRE); the cross-wave merge follows norm_held's default.
#define MI_HELD(OPC, OPN, VEC, PEEL, LPR, WPR, Q, WAVES)                                       \
    Variant{OPN "_" #VEC "_p" #PEEL "_l" #LPR "_w" #WPR "_q" #Q "_b" #WAVES,                  \
            mi_norm_variant_info{OPC, VEC, PEEL, 0, LPR, WPR, Q, WAVES,                         \
                                 (WPR == 1) ? WAVES * (64 / LPR) : WAVES / WPR,                 \
                                 (int64_t)VEC * LPR * WPR * Q, (VEC == 4 && !PEEL) ? 1 : 0},    \
            reinterpret_cast<const void *>(&norm_held<kop(OPC), VEC, (PEEL != 0), LPR, WPR, Q,  \
                                                      WAVES, true, true, 0, -1, kres(OPC)>)}

// the same shape with 4 and with 16 waves per workgroup
#define MI_HELD2(OPC, OPN, VEC, PEEL, LPR, WPR, Q, WSMALL)                                     \
    MI_HELD(OPC, OPN, VEC, PEEL, LPR, WPR, Q, WSMALL), MI_HELD(OPC, OPN, VEC, PEEL, LPR, WPR, Q, 16)

#define MI_LOOP(OPC, OPN, VEC, WAVES, U)                                                       \
    Variant{OPN "_" #VEC "_loop_b" #WAVES "_u" #U,                                              \
            mi_norm_variant_info{OPC, VEC, 0, 1, 64, WAVES, U, WAVES, 1, kUnbounded,            \
                                 VEC == 4 ? 1 : 0},                                             \
            reinterpret_cast<const void *>(&norm_looped<kop(OPC), VEC, WAVES, U, kres(OPC)>)}

// every (waves per row, slots) pair of a 128-bit path: slots 1, 2, 3, 4, 6, 8
// for 1, 2, 4, 8 and 16 waves per row
#define MI_SLOTS(OPC, OPN, PEEL, WPR, WSMALL)                                                  \
    MI_HELD2(OPC, OPN, 4, PEEL, 64, WPR, 1, WSMALL), MI_HELD2(OPC, OPN, 4, PEEL, 64, WPR, 2, WSMALL), \
    MI_HELD2(OPC, OPN, 4, PEEL, 64, WPR, 3, WSMALL), MI_HELD2(OPC, OPN, 4, PEEL, 64, WPR, 4, WSMALL), \
    MI_HELD2(OPC, OPN, 4, PEEL, 64, WPR, 6, WSMALL), MI_HELD2(OPC, OPN, 4, PEEL, 64, WPR, 8, WSMALL)
#define MI_SLOTS16(OPC, OPN, PEEL)                                                             \
    MI_HELD(OPC, OPN, 4, PEEL, 64, 16, 1, 16), MI_HELD(OPC, OPN, 4, PEEL, 64, 16, 2, 16),        \
    MI_HELD(OPC, OPN, 4, PEEL, 64, 16, 3, 16), MI_HELD(OPC, OPN, 4, PEEL, 64, 16, 4, 16),        \
    MI_HELD(OPC, OPN, 4, PEEL, 64, 16, 6, 16), MI_HELD(OPC, OPN, 4, PEEL, 64, 16, 8, 16)
#define MI_PATH128(OPC, OPN, PEEL)                                                             \
    MI_SLOTS(OPC, OPN, PEEL, 1, 4), MI_SLOTS(OPC, OPN, PEEL, 2, 4), MI_SLOTS(OPC, OPN, PEEL, 4, 4), \
    MI_SLOTS(OPC, OPN, PEEL, 8, 8), MI_SLOTS16(OPC, OPN, PEEL)

#define MI_OP_TABLE(OPC, OPN)                                                                  \
    /* 128-bit, aligned, d % 4 == 0; 16 or 32 lanes per row for narrow rows */                  \
    MI_HELD2(OPC, OPN, 4, 0, 16, 1, 1, 4), MI_HELD2(OPC, OPN, 4, 0, 32, 1, 1, 4),               \
    MI_PATH128(OPC, OPN, 0),                                                                    \
    /* 128-bit body with a per-row scalar head and tail: any d, rows congruent mod 16 B */      \
    MI_PATH128(OPC, OPN, 1),                                                                    \
    /* 32-bit accesses: any d, any 4-byte alignment */                                          \
    MI_HELD2(OPC, OPN, 1, 0, 16, 1, 1, 4), MI_HELD2(OPC, OPN, 1, 0, 32, 1, 1, 4),               \
    MI_HELD2(OPC, OPN, 1, 0, 64, 1, 1, 4), MI_HELD2(OPC, OPN, 1, 0, 64, 1, 2, 4),               \
    MI_HELD2(OPC, OPN, 1, 0, 64, 1, 4, 4), MI_HELD2(OPC, OPN, 1, 0, 64, 1, 8, 4),               \
    MI_HELD2(OPC, OPN, 1, 0, 64, 4, 4, 4), MI_HELD2(OPC, OPN, 1, 0, 64, 4, 8, 4),               \
    MI_HELD2(OPC, OPN, 1, 0, 64, 8, 8, 8),                                                      \
    MI_HELD(OPC, OPN, 1, 0, 64, 16, 8, 16), MI_HELD(OPC, OPN, 1, 0, 64, 16, 16, 16),            \
    /* streamed rows, any width */                                                             \
    MI_LOOP(OPC, OPN, 4, 4, 4), MI_LOOP(OPC, OPN, 1, 4, 8)

const Variant kVariants[] = {
    MI_OP_TABLE(MI_NORM_OP_LAYERNORM, "ln"),
    MI_OP_TABLE(MI_NORM_OP_RMSNORM, "rms"),
    MI_OP_TABLE(MI_NORM_OP_ADD_LAYERNORM, "addln"),
    MI_OP_TABLE(MI_NORM_OP_ADD_RMSNORM, "addrms"),
};
constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));

// grid cap of the grid-stride (streamed-row and copy) kernels
constexpr int64_t kMaxGrid = 1 << 20;
// row groups per launch of a held-row kernel
constexpr int64_t kMaxRowGroups = int64_t(1) << 30;

inline bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool al4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline uintptr_t addr(const void *p) { return reinterpret_cast<uintptr_t>(p); }

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

// (lanes per row, waves per row, slots) of a 32-bit row of n elements
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

// the [rows, d] row pointers a problem touches: x, r, y, h (absent ones null)
struct Rows {
    const void *p[4];
};

Rows rows_of(const mi_norm_problem &P) {
    return Rows{{P.x, kres(P.op) ? P.r : nullptr, P.y, kres(P.op) ? P.h : nullptr}};
}

struct Layout {
    bool a16;      // every row pointer and parameter 16-byte aligned, d % 4 == 0
    bool peel_ok;  // every row pointer has the same phase within 16 bytes
};

Layout layout_of(const mi_norm_problem &P) {
    const Rows R = rows_of(P);
    Layout L{P.d % 4 == 0 && al16(P.params0) && (kop(P.op) == OP_RMS || al16(P.params1)), true};
    for (const void *q : R.p) {
        if (!q) continue;
        L.a16 = L.a16 && al16(q);
        L.peel_ok = L.peel_ok && ((addr(q) ^ addr(P.x)) & 15u) == 0;
    }
    return L;
}

// the shape checks every entry point and the variant queries share
bool shape_ok(const mi_norm_problem &P) {
    if (P.op < 0 || P.op >= kOps) return false;
    if (!P.x || !P.y || !P.params0 || (kop(P.op) == OP_LN && !P.params1) || (kres(P.op) && !P.r))
        return false;
    const Rows R = rows_of(P);
    for (const void *q : R.p)
        if (q && !al4(q)) return false;
    if (!al4(P.params0) || (kop(P.op) == OP_LN && !al4(P.params1))) return false;
    if (P.d < 1 || P.d > INT32_MAX || P.rows < 0) return false;
    if (P.rows > 0 && P.rows > (INT64_MAX / (int64_t)sizeof(float)) / P.d) return false;
    return true;
}

int select_variant(const mi_norm_problem &P) {
    if (!shape_ok(P)) return -1;
    const Layout L = layout_of(P);
    const int64_t d = P.d, rows = P.rows;
    int lpr, wpr, q;
    if (L.a16) {
        const int64_t nvec = d / 4;
        if (nvec <= 16) return find(P.op, rows, 4, 0, 0, 16, 1, 1);
        if (nvec <= 32) return find(P.op, rows, 4, 0, 0, 32, 1, 1);
        shape128(nvec, rows, wpr, q);
        if (wpr) return find(P.op, rows, 4, 0, 0, 64, wpr, q);
        return find(P.op, rows, 4, 0, 1, 0, 0, 0);
    }
    if (L.peel_ok && d >= 256) {
        shape128((d + 3) / 4, rows, wpr, q);
        if (wpr) return find(P.op, rows, 4, 1, 0, 64, wpr, q);
        return find(P.op, rows, 1, 0, 1, 0, 0, 0);
    }
    ladder1(d, lpr, wpr, q);
    if (wpr) return find(P.op, rows, 1, 0, 0, lpr, wpr, q);
    return find(P.op, rows, 1, 0, 1, 0, 0, 0);
}

bool eligible(int id, const mi_norm_problem &P) {
    if (id < 0 || id >= kNumVariants || !shape_ok(P)) return false;
    const mi_norm_variant_info &v = kVariants[id].info;
    if (v.op != P.op) return false;
    const Layout L = layout_of(P);
    if (v.looped) return v.vec == 1 || L.a16;
    if (v.peel) return L.peel_ok && (P.d + 3) / 4 <= v.max_d / 4;
    if (v.vec == 4) return L.a16 && P.d <= v.max_d;
    return P.d <= v.max_d;
}

// [a, a + na) and [b, b + nb) (in floats) intersect
bool ranges_meet(const void *a, int64_t na, const void *b, int64_t nb) {
    const uintptr_t pa = addr(a), pb = addr(b);
    return pa < pb + (uintptr_t)nb * sizeof(float) && pb < pa + (uintptr_t)na * sizeof(float);
}

// Aliasing rules: two row tensors are either the same pointer or disjoint,
// the two outputs y and h never share memory, and no output overlaps a
// parameter vector (the parameters are read after earlier outputs are stored).
bool aliasing_ok(const mi_norm_problem &P) {
    if (P.rows == 0) return true;
    const int64_t n = P.rows * P.d;
    const Rows R = rows_of(P);
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j) {
            if (!R.p[i] || !R.p[j]) continue;
            if (R.p[i] == R.p[j]) {
                if (i == 2 && j == 3) return false;  // y == h
                continue;
            }
            if (ranges_meet(R.p[i], n, R.p[j], n)) return false;
        }
    for (int o = 2; o < 4; ++o) {
        if (!R.p[o]) continue;
        if (ranges_meet(R.p[o], n, P.params0, P.d)) return false;
        if (kop(P.op) == OP_LN && ranges_meet(R.p[o], n, P.params1, P.d)) return false;
    }
    return true;
}

mi_norm_status validate(const mi_norm_problem &P, float eps, const float *mean, const float *rstd) {
    if (!shape_ok(P)) return MI_NORM_ERR_INVALID;
    if (!(eps >= 0.f)) return MI_NORM_ERR_INVALID;  // also rejects NaN
    if ((mean && !al4(mean)) || (rstd && !al4(rstd))) return MI_NORM_ERR_INVALID;
    if (!aliasing_ok(P)) return MI_NORM_ERR_INVALID;
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
        const int64_t off = r0 * (int64_t)P.d;
        arg.rows = n;
        arg.x = P.x + off;
        arg.y = P.y + off;
        if (P.r) arg.r = P.r + off;
        if (P.h) arg.h = P.h + off;
        if (P.mean) arg.mean = P.mean + r0;
        if (P.rstd) arg.rstd = P.rstd + r0;
        void *args[] = {&arg};
        const int64_t blocks = (n + rpb - 1) / rpb;
        if (hipLaunchKernel(v.fn, dim3((unsigned)blocks), block, args, 0, stream) != hipSuccess)
            return MI_NORM_ERR_HIP;
    }
    return MI_NORM_OK;
}

mi_norm_problem make_problem(int op, int64_t rows, int64_t d, const float *x, const float *r,
                             const float *y, const float *h, const float *p0, const float *p1) {
    mi_norm_problem P;
    P.op = op;
    P.rows = rows;
    P.d = d;
    P.x = x;
    P.r = r;
    P.y = y;
    P.h = h;
    P.params0 = p0;
    P.params1 = p1;
    return P;
}

mi_norm_status run(int forced, const mi_norm_problem &Pb, float eps, float *mean, float *rstd,
                   hipStream_t stream) {
    const mi_norm_status st = validate(Pb, eps, mean, rstd);
    if (st != MI_NORM_OK) return st;
    int id = forced;
    if (id < 0) {
        id = select_variant(Pb);
        if (id < 0) return MI_NORM_ERR_INVALID;
    } else if (!eligible(id, Pb)) {
        return MI_NORM_ERR_INVALID;
    }
    if (Pb.rows == 0) return MI_NORM_OK;
    NormParams K;
    K.x = static_cast<const float *>(Pb.x);
    K.p0 = static_cast<const float *>(Pb.params0);
    K.p1 = static_cast<const float *>(Pb.params1);
    K.y = static_cast<float *>(const_cast<void *>(Pb.y));
    K.mean = kop(Pb.op) == OP_LN ? mean : nullptr;
    K.rstd = rstd;
    K.r = kres(Pb.op) ? static_cast<const float *>(Pb.r) : nullptr;
    K.h = kres(Pb.op) ? static_cast<float *>(const_cast<void *>(Pb.h)) : nullptr;
    K.rows = Pb.rows;
    K.d = (int32_t)Pb.d;
    K.eps = eps;
    K.inv_d = (float)(1.0 / (double)Pb.d);
    return launch(id, K, stream);
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

const char *mi_norm_version(void) { return "mi_norm 0.2.0 gfx950"; }

mi_norm_status mi_layernorm_fwd(const float *x, const float *gamma, const float *beta, float *y,
                                int64_t rows, int64_t d, float eps, float *mean, float *rstd,
                                hipStream_t stream) {
    return run(-1, make_problem(MI_NORM_OP_LAYERNORM, rows, d, x, nullptr, y, nullptr, gamma, beta),
               eps, mean, rstd, stream);
}

mi_norm_status mi_rmsnorm_fwd(const float *x, const float *w, float *y, int64_t rows, int64_t d,
                              float eps, float *rstd, hipStream_t stream) {
    return run(-1, make_problem(MI_NORM_OP_RMSNORM, rows, d, x, nullptr, y, nullptr, w, nullptr),
               eps, nullptr, rstd, stream);
}

mi_norm_status mi_add_layernorm_fwd(const float *x, const float *r, const float *gamma,
                                    const float *beta, float *y, float *h, int64_t rows, int64_t d,
                                    float eps, float *mean, float *rstd, hipStream_t stream) {
    return run(-1, make_problem(MI_NORM_OP_ADD_LAYERNORM, rows, d, x, r, y, h, gamma, beta), eps,
               mean, rstd, stream);
}

mi_norm_status mi_add_rmsnorm_fwd(const float *x, const float *r, const float *w, float *y, float *h,
                                  int64_t rows, int64_t d, float eps, float *rstd,
                                  hipStream_t stream) {
    return run(-1, make_problem(MI_NORM_OP_ADD_RMSNORM, rows, d, x, r, y, h, w, nullptr), eps,
               nullptr, rstd, stream);
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

int mi_norm_select(const mi_norm_problem *p) { return p ? select_variant(*p) : -1; }

int mi_norm_eligible(int id, const mi_norm_problem *p) { return (p && eligible(id, *p)) ? 1 : 0; }

mi_norm_status mi_layernorm_fwd_variant(int id, const float *x, const float *gamma, const float *beta,
                                        float *y, int64_t rows, int64_t d, float eps, float *mean,
                                        float *rstd, hipStream_t stream) {
    if (id < 0 || id >= kNumVariants) return MI_NORM_ERR_INVALID;
    return run(id, make_problem(MI_NORM_OP_LAYERNORM, rows, d, x, nullptr, y, nullptr, gamma, beta),
               eps, mean, rstd, stream);
}

mi_norm_status mi_rmsnorm_fwd_variant(int id, const float *x, const float *w, float *y, int64_t rows,
                                      int64_t d, float eps, float *rstd, hipStream_t stream) {
    if (id < 0 || id >= kNumVariants) return MI_NORM_ERR_INVALID;
    return run(id, make_problem(MI_NORM_OP_RMSNORM, rows, d, x, nullptr, y, nullptr, w, nullptr), eps,
               nullptr, rstd, stream);
}

mi_norm_status mi_add_layernorm_fwd_variant(int id, const float *x, const float *r, const float *gamma,
                                            const float *beta, float *y, float *h, int64_t rows,
                                            int64_t d, float eps, float *mean, float *rstd,
                                            hipStream_t stream) {
    if (id < 0 || id >= kNumVariants) return MI_NORM_ERR_INVALID;
    return run(id, make_problem(MI_NORM_OP_ADD_LAYERNORM, rows, d, x, r, y, h, gamma, beta), eps,
               mean, rstd, stream);
}

mi_norm_status mi_add_rmsnorm_fwd_variant(int id, const float *x, const float *r, const float *w,
                                          float *y, float *h, int64_t rows, int64_t d, float eps,
                                          float *rstd, hipStream_t stream) {
    if (id < 0 || id >= kNumVariants) return MI_NORM_ERR_INVALID;
    return run(id, make_problem(MI_NORM_OP_ADD_RMSNORM, rows, d, x, r, y, h, w, nullptr), eps,
               nullptr, rstd, stream);
}

mi_norm_status mi_copy_f32(const float *src, float *dst, int64_t n, hipStream_t stream) {
    if (n < 0) return MI_NORM_ERR_INVALID;
    if (n == 0) return MI_NORM_OK;
    if (!src || !dst || !al4(src) || !al4(dst)) return MI_NORM_ERR_INVALID;
    if (n > INT64_MAX / (int64_t)sizeof(float)) return MI_NORM_ERR_INVALID;
    if (ranges_meet(src, n, dst, n)) return MI_NORM_ERR_INVALID;
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
