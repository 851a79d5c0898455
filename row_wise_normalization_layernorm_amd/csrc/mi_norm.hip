// mi_norm.hip — libmi_norm.so: dispatch, validation and the C ABI declared in
// include/mi_norm.h (and the tuning calls of include/mi_norm_tuning.h) over the variant tables of variants_{f32,f16,bf16}.hip.
//
// Width dispatch mirrors the role the pages give it (mage issue #54,
// "LayerNorm [4096,768] is about 10% behind Triton's kernel": the row kernel
// covered widths up to a cap, a pair kernel the next range, and wide rows fell
// back; the fallback cost 41% at 4096 until the cap was raised).  Here every
// width has a held-row variant up to 32768 float32 elements (65536 of a
// 16-bit type: the 16-byte vector path), beyond
// which a streamed-row kernel takes over, and widths that are not a multiple
// of the vector width keep vector access through a per-row peel instead of a scalar
// fallback ("Rewriting the layer norm and matmul kernels": the scalar kernel
// stayed for those widths).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstring>

#include "mi_norm_tuning.h"
#include "norm_kernels.hpp"
#include "host_common.hpp"
#include "variant_table.hpp"

using namespace minorm;
using namespace minorm::host;

namespace minorm {

// ---------------------------------------------------------------------------
// Streaming copy (calibration): every lane moves Q 128-bit words, all loads
// before any store, the grid covering the array once, with the same
// non-temporal hints as the normalization kernels.  The shape is picked by
// size in mi_copy_f32.
template <int BLOCK, int Q>
__global__ __launch_bounds__(BLOCK)
void copy_cover(const float *src, float *dst, int64_t n4)
{
    const int64_t base = (int64_t)blockIdx.x * BLOCK * Q + threadIdx.x;
    f4 v[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int64_t i = base + (int64_t)BLOCK * q;
        v[q] = i < n4 ? ld4<true>(src + 4 * i) : f4(0.f);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int64_t i = base + (int64_t)BLOCK * q;
        if (i < n4) st4<true>(dst + 4 * i, v[q]);
    }
}

// the grid-stride form, for arrays too long for one covering grid
template <int U>
__global__ __launch_bounds__(256)
void copy_f4(const float *src, float *dst, int64_t n4)
{
    const int64_t stride = (int64_t)gridDim.x * 256 * U;
    for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n4; base += stride) {
        f4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + 256 * u;
            v[u] = i < n4 ? ld4<true>(src + 4 * i) : f4(0.f);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + 256 * u;
            if (i < n4) st4<true>(dst + 4 * i, v[u]);
        }
    }
}

// The floor of a launch (calibration): a kernel with no work, one that only
// reads (Q non-temporal 16-byte loads per lane, the sum written only when a
// flag the host never sets is set, so the loads stay), and one that only
// writes (Q non-temporal 16-byte stores per lane).  Together with the copy
// they split a normalization launch's time into launch, read and write.
__global__ __launch_bounds__(1024)
void calib_empty() {}

template <int BLOCK, int Q>
__global__ __launch_bounds__(BLOCK)
void read_cover(const float *src, float *sink, int64_t n4, int flag)
{
    const int64_t base = (int64_t)blockIdx.x * BLOCK * Q + threadIdx.x;
    f4 v[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int64_t i = base + (int64_t)BLOCK * q;
        v[q] = i < n4 ? ld4<true>(src + 4 * i) : f4(0.f);
    }
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) s += hsum(v[q]);
    if (flag) sink[(int64_t)blockIdx.x * BLOCK + threadIdx.x] = s;
}

template <int BLOCK, int Q>
__global__ __launch_bounds__(BLOCK)
void write_cover(float *dst, int64_t n4, float value)
{
    const int64_t base = (int64_t)blockIdx.x * BLOCK * Q + threadIdx.x;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int64_t i = base + (int64_t)BLOCK * q;
        if (i < n4) st4<true>(dst + 4 * i, f4(value));
    }
}

__global__ __launch_bounds__(256)
void copy_f1(const float *src, float *dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace minorm

namespace {

// grid cap of the grid-stride (streamed-row and copy) kernels
constexpr int64_t kMaxGrid = 1 << 20;
// row groups per launch of a held-row kernel
constexpr int64_t kMaxRowGroups = int64_t(1) << 30;

// Fewest workgroups that still cover every CU evenly: of the variants with
// this shape, the one with the most waves per workgroup whose grid has at
// least min_blocks(wpr) workgroups and spreads evenly over the 256 CUs;
// failing that, the one with the most workgroups.  Rows of one wave need one
// workgroup per CU (256); rows of several waves share one barrier per
// workgroup, and 16-wave workgroups only paid off with two of them per CU
// (512).  A grid whose busiest CU would hold more than 15% over the average
// is uneven: 384 16-wave workgroups (LayerNorm and RMSNorm [6144,768] float32,
// 1.5 per CU) ran 8.2 us against 7.1-7.3 us for 1536 4-wave ones.
int64_t min_blocks(int wpr) { return wpr > 1 ? 512 : 256; }
bool even_spread(int64_t blocks) {
    const int64_t per = (blocks + 255) / 256;      // workgroups on the busiest CU
    return per * 256 * 100 <= blocks * 115;
}

int find(int op, int dtype, int64_t rows, int vec, int peel, int looped, int lpr, int wpr, int q,
         int64_t min_grid = 0) {
    const int64_t need = min_grid ? min_grid : min_blocks(wpr);
    const VariantTable &T = table(dtype);
    const int base = table_base(dtype);
    int best = -1, fallback = -1;
    int64_t fallback_blocks = -1;
    for (int i = 0; i < T.n; ++i) {
        const mi_norm_variant_info &v = T.v[i].info;
        if (v.op != op || v.vec != vec || v.peel != peel || v.looped != looped) continue;
        if (v.rows_per_lane != 1) continue;
        if (looped) return base + i;
        if (v.lanes_per_row != lpr || v.waves_per_row != wpr || v.slots != q) continue;
        const int64_t blocks = (rows + v.rows_per_block - 1) / v.rows_per_block;
        if (blocks >= need && even_spread(blocks) &&
            (best < 0 || v.waves_per_block > T.v[best].info.waves_per_block))
            best = i;
        if (blocks > fallback_blocks) {
            fallback = i;
            fallback_blocks = blocks;
        }
    }
    const int pick = best >= 0 ? best : fallback;
    return pick >= 0 ? base + pick : -1;
}

// Whether the multi-row variant of an aligned vector shape should run
// (measured on MI355X against the one-row variant of the same shape; 16-bit
// rows of one or two waves are settled before this test):
// - from 8192 rows or 64 MiB of input rows: 3-17% faster (most for 16-bit
//   rows, whose parameter fetches are four times their own bytes); at 1024
//   rows it was up to 17% slower, and at 4096 rows of 16-32 MiB it went
//   either way;
// - the fused operations from 4096 rows: their one-row 16-wave workgroups
//   carry four row streams each, and two rows per wave group with 4-wave
//   workgroups ran 2-16% faster (add + LayerNorm [4096,768] float32: 8.9
//   against 10.6 us);
// - one wave per row on rows 3.5 KiB or more apart (the widest row stride,
//   in bytes): the one-row 16-wave workgroups ran 5-39% slower ([4096,1024]:
//   7.8 against 6.5 us; [4096,768] at stride 1024: 6.5 against 5.5 us),
//   while contiguous 3 KiB rows are 2-3% faster with the one-row variant;
// - never for fused float32 rows at 8 waves per row: 3-5% slower
//   ([32768,8192]), since four row streams share each parameter fetch and
//   the shared fetch saves little.
// Fused rows of four or eight waves from 8192 rows are settled before this
// test (the one-row kernel with twice the waves).
bool multi_pays(int op, int64_t rows, int64_t d, int64_t es, int wpr, int64_t pitch) {
    if (kres(op) && es == 4 && wpr >= 8) return false;
    if (rows >= 8192 || rows * d * es >= (int64_t(64) << 20)) return true;
    if (kres(op) && rows >= 4096) return true;
    return wpr == 1 && pitch >= 3584;
}


// the one-row vector variant of (wpr, q) with `waves` waves per workgroup, or -1
int find_waves(int op, int dtype, int vec, int wpr, int q, int waves) {
    const VariantTable &T = table(dtype);
    const int base = table_base(dtype);
    for (int i = 0; i < T.n; ++i) {
        const mi_norm_variant_info &v = T.v[i].info;
        if (v.op == op && v.rows_per_lane == 1 && v.vec == vec && !v.peel && !v.looped && v.lanes_per_row == 64 &&
            v.waves_per_row == wpr && v.slots == q && v.waves_per_block == waves)
            return base + i;
    }
    return -1;
}

int find_multi(int op, int dtype, int vec, int wpr, int q) {
    const VariantTable &T = table(dtype);
    const int base = table_base(dtype);
    for (int i = 0; i < T.n; ++i) {
        const mi_norm_variant_info &v = T.v[i].info;
        if (v.op == op && v.rows_per_lane == 2 && v.vec == vec && v.waves_per_row == wpr && v.slots == q)
            return base + i;
    }
    return -1;
}

// The fewest waves per row that hold it in four slots; then, while fewer
// than 4096 waves would run, twice the waves per row (from `spread_from`
// waves per row on).  Slots above six are only ever needed at 16 waves per
// row; the peeled 16-bit path has none there (max_slots 6).
void shape_vectors(int64_t nvec, int64_t rows, int &wpr, int &q, int max_slots = 8, int spread_from = 1) {
    static const int qs[] = {1, 2, 3, 4, 6, 8};
    wpr = 1;
    while (wpr < 16 && 64 * wpr * 4 < nvec) wpr *= 2;
    while (wpr < 16 && wpr >= spread_from && rows * wpr < 4096 && nvec >= 64 * 2 * wpr) wpr *= 2;
    q = pick_q(nvec, 64 * wpr, qs, max_slots >= 8 ? 6 : 5);
    if (q == 0) wpr = 0;
}

// (lanes per row, waves per row, slots) of a single-element row of n elements
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

// The row tensors a problem touches, x, r, y, h (absent ones null), with
// their row strides in elements (0 resolved to d; any stride of a one-row
// problem reads as d, since no second row is ever addressed).
struct Rows {
    const void *p[4];
    int64_t ld[4];
    bool out[4];
};

Rows rows_of(const mi_norm_problem &P) {
    const bool res = kres(P.op);
    Rows R{{P.x, res ? P.r : nullptr, P.y, res ? P.h : nullptr},
           {P.ldx, P.ldr, P.ldy, P.ldh},
           {false, false, true, true}};
    for (int i = 0; i < 4; ++i)
        if (R.ld[i] == 0 || P.rows <= 1) R.ld[i] = P.d;
    return R;
}

struct Layout {
    bool aq;         // vector path: rows and strides on 16-byte vectors, params 16 B, d % W == 0
    bool peel_ok;    // every row tensor in x's phase within a vector, on every row
    bool peel_line;  // ... and within a 128-byte cache line
};

constexpr int64_t kLine = 128;   // bytes of a cache line

Layout layout_of(const mi_norm_problem &P) {
    const Rows R = rows_of(P);
    const int64_t es = esize(P.dtype), W = vwidth(P.dtype), E = kLine / es;
    Layout L{P.d % W == 0 && al16(P.params0) && (kop(P.op) == OP_RMS || al16(P.params1)), true, true};
    const int64_t phase_x = (int64_t)((addr(P.x) / es) % W);
    const int64_t line_x = (int64_t)((addr(P.x) / es) % E);
    for (int i = 0; i < 4; ++i) {
        if (!R.p[i]) continue;
        L.aq = L.aq && al16(R.p[i]) && R.ld[i] % W == 0;
        L.peel_ok = L.peel_ok && (int64_t)((addr(R.p[i]) / es) % W) == phase_x &&
                    (R.ld[i] - R.ld[0]) % W == 0;
        L.peel_line = L.peel_line && (int64_t)((addr(R.p[i]) / es) % E) == line_x &&
                      (R.ld[i] - R.ld[0]) % E == 0;
    }
    L.peel_line = L.peel_line && L.peel_ok;
    return L;
}

// Peeled variants need a body of at least one access after a head of up to
// a cache line's elements.
constexpr int64_t kPeelMinD = 128;

// the shape checks every entry point and the variant queries share
bool shape_ok(const mi_norm_problem &P) {
    if (P.op < 0 || P.op >= kOps || P.dtype < 0 || P.dtype >= kDtypes) return false;
    if (!P.x || !P.y || !P.params0 || (kop(P.op) == OP_LN && !P.params1) || (kres(P.op) && !P.r))
        return false;
    if (P.d < 1 || P.d > kMaxD || P.rows < 0) return false;
    if (!al4(P.params0) || (kop(P.op) == OP_LN && !al4(P.params1))) return false;
    const int64_t es = esize(P.dtype);
    const int64_t raw[4] = {P.ldx, P.ldr, P.ldy, P.ldh};
    const Rows R = rows_of(P);
    for (int i = 0; i < 4; ++i) {
        if (!R.p[i]) continue;
        if (!aligned(R.p[i], (uintptr_t)es) || raw[i] < 0) return false;
        if (P.rows > 1 && R.ld[i] < P.d) return false;
        // the tensor's extent, (rows - 1) * ld + d elements, fits in int64 bytes
        if (P.rows > 1 && R.ld[i] > (INT64_MAX / es - P.d) / (P.rows - 1)) return false;
        if (P.rows == 1 && P.d > INT64_MAX / es) return false;
    }
    return true;
}

// the widest row stride of the problem's row tensors, in bytes
int64_t row_pitch(const mi_norm_problem &P) {
    const Rows R = rows_of(P);
    int64_t m = 0;
    for (int i = 0; i < 4; ++i)
        if (R.p[i] && R.ld[i] > m) m = R.ld[i];
    return m * esize(P.dtype);
}

// The aligned vector path.  A base shape, then at most one adjustment; each
// adjustment was measured on MI355X against the base (rotated buffers,
// medians of five) and kept when it won by more than the ~7% by which one
// shape varies from box to box, or when a benchmark workload takes it.
int select_vector(const mi_norm_problem &P) {
    const int op = P.op, dt = P.dtype, W = (int)vwidth(dt);
    const int64_t rows = P.rows, nvec = P.d / W;
    const bool f32 = esize(dt) == 4, res = kres(op);
    if (nvec <= 16) return find(op, dt, rows, W, 0, 0, 16, 1, 1);
    if (nvec <= 32) return find(op, dt, rows, W, 0, 0, 32, 1, 1);
    int wpr, q;
    shape_vectors(nvec, rows, wpr, q);
    if (!wpr) return find(op, dt, rows, W, 0, 1, 0, 0, 0);   // wider than any held row: streamed
    // a one-row variant of (w, s): with `waves` waves per workgroup, or by the row count
    auto one = [&](int w, int s, int waves = 0) {
        return waves ? find_waves(op, dt, W, w, s, waves) : find(op, dt, rows, W, 0, 0, 64, w, s);
    };
    auto multi = [&](int w, int s) { return find_multi(op, dt, W, w, s); };
    int v = -1;
    if (op == MI_NORM_OP_LAYERNORM && f32 && nvec > 768 && nvec <= 1024 && rows >= 3072 && rows <= 4096) {
        // float32 LayerNorm rows of 3-4 K elements: one wave of sixteen slots,
        // parameters in LDS (LayerNorm [4096,4096] 22.2 against 24.0 us)
        v = one(1, 16, rows <= 3072 ? 4 : 8);
    } else if (!f32 && wpr <= 2) {
        // 16-bit rows of one or two waves: the one-row kernel, whose
        // parameters sit in LDS (it beat the multi-row one in 12 of 15 shapes)
        if (wpr == 2 && q >= 3 && rows < 2560) {
            v = multi(2, q);   // RMSNorm BF16 [2048,4096] 6.43 against 6.84 us; add + RMSNorm 11.8 against 13.1
        } else if (res && wpr == 2 && q == 4 && rows > 4096 && rows <= 8192) {
            v = one(4, 2, 16); // fused: four waves of two slots (add + RMSNorm BF16 [8192,4096] 44.5 against 49.5 us)
        } else if (wpr == 2 && q <= 4 && rows >= 2560 && rows <= 8192) {
            // one wave with twice the slots: 4-27% ([4096,4096] RMSNorm 11.5 against
            // 13.7 us), in 4-wave workgroups where 16-wave ones spread unevenly
            const int64_t b16 = (rows + 15) / 16;
            v = one(1, 2 * q, (b16 > 256 && !even_spread(b16)) ? 4 : 16);
        } else if (wpr == 1 && !(q <= 2 && !res && rows <= 8192)) {
            v = one(1, q, 4);  // one-wave rows: 4-wave workgroups won in 6 of 8 shapes
        }
    } else if (res && (wpr == 4 || wpr == 8) && rows >= 8192) {
        // fused rows of four or eight waves, many rows: twice the waves, half the
        // slots (add + LayerNorm [16384,8192] 349 against 395 us; BF16 [32768,8192] 342 against 365)
        v = one(2 * wpr, (q + 1) / 2);
    } else if (res && f32 && wpr == 2 && nvec > 256 && rows <= 4096) {
        v = one(1, 8, 4);      // fused float32 rows of two waves: one wave of eight slots (add + LN [2048,1536] 8.89 against 9.90 us)
    } else if (res && f32 && wpr == 4 && nvec > 512 && q <= 4 && rows >= 2048 && rows < 4096) {
        v = multi(2, 2 * q);   // fused float32 rows of four waves: add + RMSNorm [2048,3072] 16.9 against 18.2 us
    } else if (multi_pays(op, rows, P.d, esize(dt), wpr, row_pitch(P))) {
        v = multi(wpr, q);     // many rows: two rows per wave group, one parameter fetch for both
    } else if (f32 && !res && (wpr == 2 || wpr == 4) && q <= 4 && rows * wpr > 8192) {
        v = one(wpr / 2, 2 * q);   // more than 4096 waves even at half the waves: 10-12%
    } else if (!f32 && wpr == 4 && q <= 4 && rows >= 2048 && (!res || rows < 2560)) {
        v = one(2, 2 * q, 16);     // 16-bit rows of four waves: 5-11%
    }
    return v >= 0 ? v : one(wpr, q);
}

int select_variant(const mi_norm_problem &P) {
    if (!shape_ok(P)) return -1;
    const Layout L = layout_of(P);
    const int op = P.op, dt = P.dtype, W = (int)vwidth(dt);
    const int64_t d = P.d, rows = P.rows;
    int lpr, wpr, q;
    if (L.aq) return select_vector(P);
    if (L.peel_ok && d >= 256) {
        // the head and tail are held apart from the body, which holds at most
        // d / W accesses.  Peeled rows, whose parameters are fetched with the
        // row, spread over more waves only from eight waves per row, and take
        // the largest workgroups that still give every CU one: at 512-2048
        // rows 10-25% faster than more waves per row in 4-wave workgroups
        // (LayerNorm [1024,2049] 4.88 against 6.10 us, RMSNorm [1024,4097]
        // 7.27 against 8.34, LayerNorm BF16 [1024,4100] 5.57 against 6.81)
        shape_vectors(d / W, rows, wpr, q, W == 8 ? 6 : 8, 8);
        return wpr ? find(op, dt, rows, W, 1, 0, 64, wpr, q, 256) : find(op, dt, rows, 1, 0, 1, 0, 0, 0);
    }
    ladder1(d, lpr, wpr, q);
    return wpr ? find(op, dt, rows, 1, 0, 0, lpr, wpr, q) : find(op, dt, rows, 1, 0, 1, 0, 0, 0);
}

bool eligible(int id, const mi_norm_problem &P) {
    const Variant *V = variant(id);
    if (!V || !shape_ok(P)) return false;
    const mi_norm_variant_info &v = V->info;
    if (v.op != P.op || v.dtype != P.dtype) return false;
    const Layout L = layout_of(P);
    if (v.looped) return v.vec == 1 || L.aq;
    if (v.peel) return L.peel_ok && P.d >= kPeelMinD && P.d <= v.max_d;
    if (v.vec > 1) return L.aq && P.d <= v.max_d;
    return P.d <= v.max_d;
}

// Aliasing rules (see the header): an output row tensor is an input row
// tensor (same pointer and stride) or shares no element with any other row
// tensor; y and h share nothing; no output meets a parameter vector; mean
// and rstd meet nothing else.
bool aliasing_ok(const mi_norm_problem &P) {
    if (P.rows == 0) return true;
    const Rows R = rows_of(P);
    const int64_t es = esize(P.dtype), rows = P.rows, d = P.d;
    const bool ln = kop(P.op) == OP_LN;
    for (int o = 2; o < 4; ++o) {
        if (!R.p[o]) continue;
        for (int t = 0; t < 4; ++t) {
            if (t == o || !R.p[t]) continue;
            if (!R.out[t] && R.p[t] == R.p[o] && R.ld[t] == R.ld[o]) continue;  // in place
            if (rows_meet(R.p[o], R.ld[o], R.p[t], R.ld[t], rows, d, es)) return false;
        }
        const Ext eo = rows_ext(R.p[o], R.ld[o], rows, d, es);
        if (meet(eo, vec_ext(P.params0, d, 4))) return false;
        if (ln && meet(eo, vec_ext(P.params1, d, 4))) return false;
    }
    float *const stats[2] = {ln ? P.mean : nullptr, P.rstd};
    for (int s = 0; s < 2; ++s) {
        if (!stats[s]) continue;
        const Ext es_ = vec_ext(stats[s], rows, 4);
        for (int t = 0; t < 4; ++t)
            if (R.p[t] && meet(es_, rows_ext(R.p[t], R.ld[t], rows, d, es))) return false;
        if (meet(es_, vec_ext(P.params0, d, 4))) return false;
        if (ln && meet(es_, vec_ext(P.params1, d, 4))) return false;
    }
    if (stats[0] && stats[1] && meet(vec_ext(stats[0], rows, 4), vec_ext(stats[1], rows, 4))) return false;
    return true;
}

mi_norm_status validate(const mi_norm_problem &P) {
    if (!shape_ok(P)) return MI_NORM_ERR_INVALID;
    if (!(P.eps >= 0.f)) return MI_NORM_ERR_INVALID;  // also rejects NaN
    const float *mean = kop(P.op) == OP_LN ? P.mean : nullptr;
    if ((mean && !al4(mean)) || (P.rstd && !al4(P.rstd))) return MI_NORM_ERR_INVALID;
    if (!aliasing_ok(P)) return MI_NORM_ERR_INVALID;
    return MI_NORM_OK;
}

// Held variants give each workgroup one row group, so the grid is
// ceil(rows / rows_per_block).  Only a row count beyond kMaxRowGroups row
// groups (2^30, far past device memory for any width) is split over several
// launches; streamed variants walk rows with a grid-stride loop.
mi_norm_status launch(const Variant &v, const NormParams &P, int64_t es, hipStream_t stream) {
    if (P.rows == 0) return MI_NORM_OK;
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
    auto adv = [&](const void *p, int64_t ld, int64_t r0) -> const char * {
        return p ? static_cast<const char *>(p) + r0 * ld * es : nullptr;
    };
    for (int64_t r0 = 0; r0 < P.rows; r0 += chunk) {
        NormParams arg = P;
        const int64_t n = (P.rows - r0) < chunk ? (P.rows - r0) : chunk;
        arg.rows = n;
        arg.x = adv(P.x, P.ldx, r0);
        arg.y = const_cast<char *>(adv(P.y, P.ldy, r0));
        arg.r = adv(P.r, P.ldr, r0);
        arg.h = const_cast<char *>(adv(P.h, P.ldh, r0));
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
                             float *y, float *h, const float *p0, const float *p1, float eps,
                             float *mean, float *rstd) {
    mi_norm_problem P;
    std::memset(&P, 0, sizeof(P));
    P.op = op;
    P.dtype = MI_NORM_F32;
    P.rows = rows;
    P.d = d;
    P.x = x;
    P.r = r;
    P.y = y;
    P.h = h;
    P.params0 = p0;
    P.params1 = p1;
    P.eps = eps;
    P.mean = mean;
    P.rstd = rstd;
    return P;
}

mi_norm_status run(int forced, const mi_norm_problem &Pb, hipStream_t stream) {
    const mi_norm_status st = validate(Pb);
    if (st != MI_NORM_OK) return st;
    int id = forced;
    if (id < 0) {
        id = select_variant(Pb);
        if (id < 0) return MI_NORM_ERR_INVALID;
    } else if (!eligible(id, Pb)) {
        return MI_NORM_ERR_INVALID;
    }
    if (Pb.rows == 0) return MI_NORM_OK;
    const Rows R = rows_of(Pb);
    NormParams K;
    K.x = R.p[0];
    K.r = R.p[1];
    K.y = const_cast<void *>(R.p[2]);
    K.h = const_cast<void *>(R.p[3]);
    K.ldx = R.ld[0];
    K.ldr = R.ld[1];
    K.ldy = R.ld[2];
    K.ldh = R.ld[3];
    K.p0 = Pb.params0;
    K.p1 = kop(Pb.op) == OP_LN ? Pb.params1 : nullptr;
    K.mean = kop(Pb.op) == OP_LN ? Pb.mean : nullptr;
    K.rstd = Pb.rstd;
    K.rows = Pb.rows;
    K.d = (int32_t)Pb.d;
    K.eps = Pb.eps;
    K.inv_d = (float)(1.0 / (double)Pb.d);
    // a peeled row's body starts on a cache line when every row tensor
    // shares its phase within one (each wave-wide access then covers whole
    // lines: 3-4% on [256,8193]), else on a 16-byte boundary
    K.peel_align = (int32_t)(layout_of(Pb).peel_line ? kLine / esize(Pb.dtype) : vwidth(Pb.dtype));
    return launch(*variant(id), K, esize(Pb.dtype), stream);
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

const char *mi_norm_version(void) { return "mi_norm 0.5.0 gfx950"; }

mi_norm_status mi_layernorm_fwd(const float *x, const float *gamma, const float *beta, float *y,
                                int64_t rows, int64_t d, float eps, float *mean, float *rstd,
                                hipStream_t stream) {
    return run(-1, make_problem(MI_NORM_OP_LAYERNORM, rows, d, x, nullptr, y, nullptr, gamma, beta, eps,
                                mean, rstd), stream);
}

mi_norm_status mi_rmsnorm_fwd(const float *x, const float *w, float *y, int64_t rows, int64_t d,
                              float eps, float *rstd, hipStream_t stream) {
    return run(-1, make_problem(MI_NORM_OP_RMSNORM, rows, d, x, nullptr, y, nullptr, w, nullptr, eps,
                                nullptr, rstd), stream);
}

mi_norm_status mi_add_layernorm_fwd(const float *x, const float *r, const float *gamma,
                                    const float *beta, float *y, float *h, int64_t rows, int64_t d,
                                    float eps, float *mean, float *rstd, hipStream_t stream) {
    return run(-1, make_problem(MI_NORM_OP_ADD_LAYERNORM, rows, d, x, r, y, h, gamma, beta, eps, mean,
                                rstd), stream);
}

mi_norm_status mi_add_rmsnorm_fwd(const float *x, const float *r, const float *w, float *y, float *h,
                                  int64_t rows, int64_t d, float eps, float *rstd,
                                  hipStream_t stream) {
    return run(-1, make_problem(MI_NORM_OP_ADD_RMSNORM, rows, d, x, r, y, h, w, nullptr, eps, nullptr,
                                rstd), stream);
}

mi_norm_status mi_norm_fwd(const mi_norm_problem *p, hipStream_t stream) {
    return p ? run(-1, *p, stream) : MI_NORM_ERR_INVALID;
}

mi_norm_status mi_norm_check(const mi_norm_problem *p) {
    if (!p) return MI_NORM_ERR_INVALID;
    const mi_norm_status st = validate(*p);
    if (st != MI_NORM_OK) return st;
    return select_variant(*p) >= 0 ? MI_NORM_OK : MI_NORM_ERR_INVALID;
}

mi_norm_status mi_norm_fwd_variant(int id, const mi_norm_problem *p, hipStream_t stream) {
    if (!p || !variant(id)) return MI_NORM_ERR_INVALID;
    return run(id, *p, stream);
}

int mi_norm_variant_count(void) { return num_variants(); }

const char *mi_norm_variant_name(int id) {
    const Variant *v = variant(id);
    return v ? v->name : nullptr;
}

mi_norm_status mi_norm_variant_get_info(int id, mi_norm_variant_info *out) {
    const Variant *v = variant(id);
    if (!v || !out) return MI_NORM_ERR_INVALID;
    *out = v->info;
    return MI_NORM_OK;
}

int mi_norm_select(const mi_norm_problem *p) { return p ? select_variant(*p) : -1; }

int mi_norm_eligible(int id, const mi_norm_problem *p) { return (p && eligible(id, *p)) ? 1 : 0; }

mi_norm_status mi_layernorm_fwd_variant(int id, const float *x, const float *gamma, const float *beta,
                                        float *y, int64_t rows, int64_t d, float eps, float *mean,
                                        float *rstd, hipStream_t stream) {
    if (!variant(id)) return MI_NORM_ERR_INVALID;
    return run(id, make_problem(MI_NORM_OP_LAYERNORM, rows, d, x, nullptr, y, nullptr, gamma, beta, eps,
                                mean, rstd), stream);
}

mi_norm_status mi_rmsnorm_fwd_variant(int id, const float *x, const float *w, float *y, int64_t rows,
                                      int64_t d, float eps, float *rstd, hipStream_t stream) {
    if (!variant(id)) return MI_NORM_ERR_INVALID;
    return run(id, make_problem(MI_NORM_OP_RMSNORM, rows, d, x, nullptr, y, nullptr, w, nullptr, eps,
                                nullptr, rstd), stream);
}

mi_norm_status mi_add_layernorm_fwd_variant(int id, const float *x, const float *r, const float *gamma,
                                            const float *beta, float *y, float *h, int64_t rows,
                                            int64_t d, float eps, float *mean, float *rstd,
                                            hipStream_t stream) {
    if (!variant(id)) return MI_NORM_ERR_INVALID;
    return run(id, make_problem(MI_NORM_OP_ADD_LAYERNORM, rows, d, x, r, y, h, gamma, beta, eps, mean,
                                rstd), stream);
}

mi_norm_status mi_add_rmsnorm_fwd_variant(int id, const float *x, const float *r, const float *w,
                                          float *y, float *h, int64_t rows, int64_t d, float eps,
                                          float *rstd, hipStream_t stream) {
    if (!variant(id)) return MI_NORM_ERR_INVALID;
    return run(id, make_problem(MI_NORM_OP_ADD_RMSNORM, rows, d, x, r, y, h, w, nullptr, eps, nullptr,
                                rstd), stream);
}

mi_norm_status mi_copy_f32(const float *src, float *dst, int64_t n, hipStream_t stream) {
    if (n < 0) return MI_NORM_ERR_INVALID;
    if (n == 0) return MI_NORM_OK;
    if (!src || !dst || !al4(src) || !al4(dst)) return MI_NORM_ERR_INVALID;
    if (n > INT64_MAX / (int64_t)sizeof(float)) return MI_NORM_ERR_INVALID;
    if (meet(vec_ext(src, n, 4), vec_ext(dst, n, 4))) return MI_NORM_ERR_INVALID;
    hipError_t e;
    if (n % 4 == 0 && al16(src) && al16(dst)) {
        // the fastest covering shape measured on MI355X for the bytes moved
        // (read + written), rotating buffers past the caches: 12.6 MB 512x3
        // (3.40 us), 25 MB 256x4 (5.25), 50 and 100 MB 256x8 (8.65, 17.0),
        // 200 MB 1024x1 (32.6), 1 and 2 GB 256x1 (164, 329)
        const int64_t n4 = n / 4, bytes = 8 * n;
        int block = 256, q = 1;
        const void *fn = reinterpret_cast<const void *>(&copy_cover<256, 1>);
        if (bytes <= (int64_t(16) << 20)) {
            block = 512, q = 3, fn = reinterpret_cast<const void *>(&copy_cover<512, 3>);
        } else if (bytes <= (int64_t(48) << 20)) {
            q = 4, fn = reinterpret_cast<const void *>(&copy_cover<256, 4>);
        } else if (bytes <= (int64_t(160) << 20)) {
            q = 8, fn = reinterpret_cast<const void *>(&copy_cover<256, 8>);
        } else if (bytes <= (int64_t(768) << 20)) {
            block = 1024, fn = reinterpret_cast<const void *>(&copy_cover<1024, 1>);
        }
        int64_t blocks = (n4 + (int64_t)block * q - 1) / ((int64_t)block * q);
        int64_t n4a = n4;
        const float *s = src;
        float *dd = dst;
        void *args[] = {&s, &dd, &n4a};
        if (blocks <= INT32_MAX) {
            e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(block), args, 0, stream);
        } else {
            blocks = kMaxGrid;
            e = hipLaunchKernel(reinterpret_cast<const void *>(&copy_f4<1>), dim3((unsigned)blocks), dim3(256),
                                args, 0, stream);
        }
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

mi_norm_status mi_calib_launch(int kind, const float *src, float *dst, int64_t n, hipStream_t stream) {
    // kind 0: one empty launch of 256 workgroups of 1024 threads (n, src,
    // dst unused); 1: read n floats from src; 2: write n floats to dst.
    // Arrays are 16-byte aligned with n % 4 == 0 and n / 4 < 2^31 * 256.
    if (kind == 0) {
        return hipLaunchKernel(reinterpret_cast<const void *>(&calib_empty), dim3(256), dim3(1024), nullptr, 0,
                               stream) == hipSuccess ? MI_NORM_OK : MI_NORM_ERR_HIP;
    }
    if ((kind != 1 && kind != 2) || n <= 0 || n % 4 != 0 || n / 4 > (int64_t)INT32_MAX * 256)
        return MI_NORM_ERR_INVALID;
    const float *p = kind == 1 ? src : dst;
    if (!p || !al16(p)) return MI_NORM_ERR_INVALID;
    int64_t n4 = n / 4;
    // the copy's shape rule on the bytes one pass moves: 512x3 up to 16 MB,
    // 256x4 up to 48 MB, 256x8 up to 160 MB, 256x1 beyond
    const int64_t bytes = 4 * n;
    int block = 256, q = 1;
    if (bytes <= (int64_t(16) << 20)) block = 512, q = 3;
    else if (bytes <= (int64_t(48) << 20)) q = 4;
    else if (bytes <= (int64_t(160) << 20)) q = 8;
    const int64_t blocks = (n4 + (int64_t)block * q - 1) / ((int64_t)block * q);
    const void *fn;
    if (kind == 1) {
        fn = block == 512 ? reinterpret_cast<const void *>(&read_cover<512, 3>)
           : q == 4 ? reinterpret_cast<const void *>(&read_cover<256, 4>)
           : q == 8 ? reinterpret_cast<const void *>(&read_cover<256, 8>)
           : reinterpret_cast<const void *>(&read_cover<256, 1>);
        const float *s_ = src;
        float *sink = nullptr;
        int flag = 0;
        void *args[] = {&s_, &sink, &n4, &flag};
        return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(block), args, 0, stream) == hipSuccess
                   ? MI_NORM_OK : MI_NORM_ERR_HIP;
    }
    fn = block == 512 ? reinterpret_cast<const void *>(&write_cover<512, 3>)
       : q == 4 ? reinterpret_cast<const void *>(&write_cover<256, 4>)
       : q == 8 ? reinterpret_cast<const void *>(&write_cover<256, 8>)
       : reinterpret_cast<const void *>(&write_cover<256, 1>);
    float *d_ = dst;
    float value = 1.f;
    void *args[] = {&d_, &n4, &value};
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(block), args, 0, stream) == hipSuccess
               ? MI_NORM_OK : MI_NORM_ERR_HIP;
}

}  // extern "C"
