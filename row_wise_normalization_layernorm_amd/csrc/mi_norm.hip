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

int find(int op, int dtype, int64_t rows, int vec, int peel, int looped, int lpr, int wpr, int q) {
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
        if (blocks >= min_blocks(wpr) && even_spread(blocks) &&
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

// Slots above six are only ever needed at 16 waves per row; the peeled
// 16-bit path has none there (max_slots 6).
void shape_vectors(int64_t nvec, int64_t rows, int &wpr, int &q, int max_slots = 8) {
    static const int qs[] = {1, 2, 3, 4, 6, 8};
    wpr = 1;
    while (wpr < 16 && 64 * wpr * 4 < nvec) wpr *= 2;
    while (wpr < 16 && rows * wpr < 4096 && nvec >= 64 * 2 * wpr) wpr *= 2;
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
    if (P.d < 1 || P.d > INT32_MAX || P.rows < 0) return false;
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

int select_variant(const mi_norm_problem &P) {
    if (!shape_ok(P)) return -1;
    const Layout L = layout_of(P);
    const int64_t d = P.d, rows = P.rows;
    const int op = P.op, dt = P.dtype;
    const int W = (int)vwidth(dt);
    int lpr, wpr, q;
    if (L.aq) {
        const int64_t nvec = d / W;
        if (nvec <= 16) return find(op, dt, rows, W, 0, 0, 16, 1, 1);
        if (nvec <= 32) return find(op, dt, rows, W, 0, 0, 32, 1, 1);
        shape_vectors(nvec, rows, wpr, q);
        if (wpr && wpr <= 2 && esize(dt) == 2) {
            // 16-bit rows of one or two waves: the one-row variants, which
            // stage their parameters in LDS, beat the multi-row ones in 12
            // of 15 measured shapes (up to 10%: LayerNorm bfloat16
            // [16384,768] 10.6 against 11.9 us).  With 2560-8192 rows, rows
            // of two waves run as one wave with twice the slots in 16-wave
            // workgroups: 4-27% faster in eight shapes (RMSNorm [4096,4096]
            // 11.5 against 13.7 us; LayerNorm [2560,4096] 8.7 against 11.0),
            // equal in one; at 12288 rows it lost 4%.  One wave of up to four
            // slots takes 4-wave workgroups (the faster in 6 of 8 shapes).
            // Under 2560 rows, rows of two waves and three or four slots
            // take the multi-row kernel of the same shape: bfloat16
            // RMSNorm [2048,4096] 6.43 against 6.84 us, LayerNorm 7.26
            // against 7.58, add + RMSNorm 11.8 against 13.1, RMSNorm
            // [2048,3072] 5.33 against more than 5.44 (two slots: LayerNorm
            // [2048,2048] lost).
            if (wpr == 2 && q >= 3 && rows < 2560) {
                const int m = find_multi(op, dt, W, 2, q);
                if (m >= 0) return m;
            }
            if (kres(op) && wpr == 2 && q == 4 && rows > 4096 && rows <= 8192) {
                // fused rows of two waves and four slots, 4097-8192 rows:
                // four waves of two slots in 16-wave workgroups (add +
                // LayerNorm bfloat16 [8000,4096] 44.3 against 48.8 us,
                // [6144,4096] 34.8 against 37.1; add + RMSNorm [5000,4096]
                // 28.3 against 29.2); at 4096 rows (24.4 against 23.1) and
                // for rows of three slots it lost
                const int s = find_waves(op, dt, W, 4, 2, 16);
                if (s >= 0) return s;
            }
            if (wpr == 2 && q <= 4 && rows >= 2560 && rows <= 8192) {
                // 4-wave workgroups where more than 256 16-wave ones would
                // spread unevenly over the CUs: bfloat16 LayerNorm
                // [5000,3000] (313 workgroups) 13.7 against 15.8 us,
                // [4500,4096] 16.0 against 17.8, RMSNorm [6144,3072] 14.4
                // against 15.7, add + LayerNorm [6144,4096] 37.1 against 40.1
                const int64_t b16 = (rows + 15) / 16;
                const int s = (b16 > 256 && !even_spread(b16)) ? find_waves(op, dt, W, 1, 2 * q, 4) : -1;
                if (s >= 0) return s;
                const int t = find_waves(op, dt, W, 1, 2 * q, 16);
                if (t >= 0) return t;
            }
            // With the buffer-load kernel, plain (not fused) rows of one or
            // two slots up to 8192 rows run faster in the workgroup rule's
            // 16-wave workgroups (LayerNorm bfloat16 [4096,768] 4.03 against
            // 4.22 us, [8192,768] 5.92 against 6.46; RMSNorm [4096,768] a
            // tie); from 16384 rows, for fused rows and for four slots the
            // 4-wave ones kept a 2-13% lead.
            const bool small = wpr == 1 && q <= 2 && !kres(op) && rows <= 8192;
            const int s = (wpr == 1 && !small) ? find_waves(op, dt, W, wpr, q, 4) : -1;
            return s >= 0 ? s : find(op, dt, rows, W, 0, 0, 64, wpr, q);
        }
        if (op == MI_NORM_OP_LAYERNORM && esize(dt) == 4 && nvec > 768 && nvec <= 1024 && rows >= 3072 &&
            rows <= 4096) {
            // float32 LayerNorm rows of 3-4 K elements, 3072-4096 of them:
            // one wave per row with sixteen slots and the parameters in LDS
            // (5 waves per SIMD), measured on MI355X as the fastest shape or
            // within 2.5% of it ([4096,4096] 22.4 us; [3072,4096] 17.7 against
            // 17.4 for 16-wave workgroups; [4096,3200] 18.1), and up to 7%
            // ahead of the one-row shapes outside it
            const int s = find_waves(op, dt, W, 1, 16, rows <= 3072 ? 4 : 8);
            if (s >= 0) return s;
        }
        if (kres(op) && (wpr == 4 || wpr == 8) && rows >= 8192) {
            // fused rows of four or eight waves with many rows: the one-row
            // kernel with twice the waves per row and half the slots.  On
            // MI355X, add + LayerNorm [32768,8192] float32 716 against 731 us,
            // bfloat16 342 against 365 (the multi-row kernel); on seven
            // further shapes faster in six by 1.7-12% ([16384,8192] 349
            // against 395 us), 1% slower at [8192,4096]
            const int s = find(op, dt, rows, W, 0, 0, 64, 2 * wpr, (q + 1) / 2);
            if (s >= 0) return s;
        }
        if (op == MI_NORM_OP_RMSNORM && esize(dt) == 4 && wpr == 4 && rows >= 8192) {
            // float32 RMSNorm rows of four waves from 8192 rows: the one-row
            // kernel with eight waves per row and half the slots, in 8-wave
            // workgroups ([32768,4096] 168.0 against 176.8 us for the
            // multi-row kernel, [16384,4096] 85.4 against 88.6, [8192,3584]
            // 39.4 against 39.8, [12288,3072] 49.8 against 50.1; 16-wave
            // workgroups lost 2-5%)
            const int s = find_waves(op, dt, W, 8, (q + 1) / 2, 8);
            if (s >= 0) return s;
        }
        if (kres(op) && esize(dt) == 4 && wpr == 2 && nvec > 256 && rows <= 4096) {
            // fused float32 rows of two waves by width (more than 256
            // quads, not doubled for few rows), up to 4096 rows: one wave of
            // eight slots in 4-wave workgroups (add + LayerNorm [2048,1536]
            // 8.82 against 10.2 us, [4096,2048] 23.0 against 24.7 for the
            // multi-row kernel, [2048,2048] 11.6 against 12.3; add + RMSNorm
            // [3072,2048] 16.9 against 18.2, [4096,1536] 16.8 against 17.5);
            // eight slots beat six for rows of six ([2048,1536] 8.82 against
            // 9.31); at 6144 rows the multi-row kernel tied
            const int s = find_waves(op, dt, W, 1, 8, 4);
            if (s >= 0) return s;
        }
        if (kres(op) && esize(dt) == 4 && wpr == 4 && nvec > 512 && q <= 4 && rows >= 2048 && rows < 4096) {
            // fused float32 rows of four waves by width, 2048-4095 rows: the
            // multi-row kernel with two waves per row and twice the slots
            // (add + LayerNorm [3000,3000] 26.8 against 29.3 us, add +
            // RMSNorm [2048,3072] 16.9 against 18.2)
            const int m = find_multi(op, dt, W, 2, 2 * q);
            if (m >= 0) return m;
        }
        if (op == MI_NORM_OP_RMSNORM && esize(dt) == 4 && wpr == 2 && nvec > 256 && rows >= 2048 &&
            rows <= 4096) {
            // float32 RMSNorm rows of two waves by width, 2048-4096 rows:
            // the multi-row kernel of the same shape ([2560,2048] 7.55
            // against 7.94 us, [2048,2048] 6.41 against 6.70, [4096,1536]
            // 8.63 against 8.96, [4096,2048] 11.79 against 11.88); LayerNorm
            // tied or lost there ([4096,2048] 13.2 against 11.5)
            const int m = find_multi(op, dt, W, 2, q);
            if (m >= 0) return m;
        }
        if (wpr && multi_pays(op, rows, d, esize(dt), wpr, row_pitch(P))) {
            if (op == MI_NORM_OP_LAYERNORM && esize(dt) == 4 && (wpr == 2 || wpr == 4) && rows >= 8192 &&
                (q * wpr) % 8 == 0) {
                // float32 LayerNorm rows of two or four waves from 8192 rows,
                // whose slots split evenly over eight waves: eight waves per
                // row with as many fewer slots ([16384,4096] 88.8 against
                // 91.1 us, [32768,2048] 86.0 against 88.9 or more, [65536,2048]
                // 171 against 186; ties at [8192,2048]).  Splits that leave
                // slots idle ([16384,2560]: three slots of four waves) lost
                // 3-4%.
                const int m = find_multi(op, dt, W, 8, q * wpr / 8);
                if (m >= 0) return m;
            }
            const int m = find_multi(op, dt, W, wpr, q);
            if (m >= 0) return m;
        }
        if (esize(dt) == 4 && !kres(op) && (wpr == 2 || wpr == 4) && q <= 4 && rows * (wpr / 2) > 4096) {
            // float32 rows of 2-4 K elements on the one-row path with more
            // than 4096 waves at half the waves per row: half the waves, twice
            // the slots, one fewer cross-wave exchange ([2560,4096] 14.6
            // against 16.2 us; [4096,3072] 17.1 against 19.5; [6144,2048]
            // 17.3 against 19.5; at [2048,4096] four waves stay 2% ahead)
            wpr /= 2;
            q *= 2;
        }
        if (esize(dt) == 2 && wpr == 4 && q <= 4 && rows >= 2048 && (!kres(op) || rows < 2560)) {
            // 16-bit rows of four waves on the one-row path from 2048 rows:
            // two waves with twice the slots in 16-wave workgroups (bfloat16
            // LayerNorm [2048,4608] 8.18 against 9.07 us, [4096,6144] 19.5
            // against 21.4, [2048,8192] 12.9 against 13.6; RMSNorm
            // [2048,8192] 12.1 against 13.5, [4096,6144] 17.8 against more
            // than 19.5; add + RMSNorm [2048,8192] 23.3 against 24.5); at
            // 1024 rows it lost, and fused rows from 2560 rows lost 5-15%
            // (add + RMSNorm [3000,6000] 31.6 against 27.5 us)
            const int s = find_waves(op, dt, W, 2, 2 * q, 16);
            if (s >= 0) return s;
        }
        if (wpr) return find(op, dt, rows, W, 0, 0, 64, wpr, q);
        return find(op, dt, rows, W, 0, 1, 0, 0, 0);
    }
    if (L.peel_ok && d >= 256) {
        // the head and tail are held apart from the body, which holds at
        // most d / W accesses
        shape_vectors(d / W, rows, wpr, q, W == 8 ? 6 : 8);
        if (wpr) return find(op, dt, rows, W, 1, 0, 64, wpr, q);
        return find(op, dt, rows, 1, 0, 1, 0, 0, 0);
    }
    ladder1(d, lpr, wpr, q);
    if (wpr) return find(op, dt, rows, 1, 0, 0, lpr, wpr, q);
    return find(op, dt, rows, 1, 0, 1, 0, 0, 0);
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
