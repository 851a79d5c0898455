// bwd_kernels.hpp — gfx950 device code for the LayerNorm / RMSNorm backward.
//
// Given the upstream gradient dy, the input x, gamma (or w) and the forward's
// per-row statistics, per row i with xhat = (x - mu) * rstd (RMSNorm: x * rstd)
// and g = dy * gamma:
//     dx = rstd * (g - mean_j(g) - xhat * mean_j(g * xhat))       (LayerNorm)
//     dx = rstd * (g - xhat * mean_j(g * xhat))                    (RMSNorm)
// and over all rows dgamma_j = sum_i dy_ij xhat_ij, dbeta_j = sum_i dy_ij.
//
// The row part has the forward's shape: a row held in registers by WPR
// waves, its two sums met through DPP and (WPR > 1) one LDS exchange, dx
// stored from the same registers.  The column part is a reduction across
// rows, so a lane keeps the same columns for every row its workgroup visits
// (a grid-stride loop over row groups) and adds its terms into float64
// registers; at the end the row slots of the workgroup meet in an LDS tree
// and the workgroup writes one float32 partial row; a second kernel sums the
// partial rows in float64 in a fixed order (deterministic results).
// Rows wider than the held variants take a streamed path: per-row sums first
// (one workgroup per row), then a two-dimensional grid of column chunks by
// row blocks that computes dx and the partial sums.
#pragma once

#include "norm_kernels.hpp"

namespace minorm {

typedef double d4 __attribute__((ext_vector_type(4)));
typedef double d8 __attribute__((ext_vector_type(8)));
template <int VEC> struct DVecOf;
template <> struct DVecOf<1> { using type = double; };
template <> struct DVecOf<4> { using type = d4; };
template <> struct DVecOf<8> { using type = d8; };
template <int VEC> using vd = typename DVecOf<VEC>::type;

template <int VEC>
__device__ __forceinline__ vd<VEC> widen64(vf<VEC> v) {
    if constexpr (VEC == 1) return (double)v;
    else return __builtin_convertvector(v, vd<VEC>);
}
template <int VEC>
__device__ __forceinline__ vf<VEC> narrow32(vd<VEC> v) {
    if constexpr (VEC == 1) return (float)v;
    else return __builtin_convertvector(v, vf<VEC>);
}

// VEC float32 values stored to consecutive addresses (partial rows)
template <int VEC>
__device__ __forceinline__ void stp(float *p, vf<VEC> v) {
    if constexpr (VEC == 1) {
        *p = v;
    } else if constexpr (VEC == 4) {
        st4<false>(p, v);
    } else {
        st4<false>(p, v.lo);
        st4<false>(p + 4, v.hi);
    }
}

struct BwdParams {
    const void *dy;
    const void *x;
    void *dx;
    const float *p0;      // gamma (LayerNorm) or w (RMSNorm)
    const float *mean;    // LayerNorm only
    const float *rstd;
    float *part;          // partial parameter gradients [blocks][NG][dpad], or null: not wanted
    float2 *stats;        // streamed path: (mean_j g, mean_j g xhat) per row
    int64_t rows;
    int64_t lddy, ldx, lddx;
    int32_t d;
    int32_t dpad;         // partial row pitch: d rounded up to a multiple of 4
    float inv_d;
};

// ---------------------------------------------------------------------------
// Held rows.
//   T      storage type of dy, x, dx
//   OP     OP_LN or OP_RMS
//   VEC    elements per access: 4 (float32) / 8 (16-bit) with aligned rows, or 1
//   WPR    waves per row; WAVES / WPR rows per workgroup per step (1, 2, 4, 8)
//   Q      accesses held per lane; capacity VEC * 64 * WPR * Q elements
// Lane li of wave rank wr holds access k = li + 64 * (wr + WPR * q) of every
// row its row slot visits.
template <typename T, int OP, int VEC, int WPR, int Q, int WAVES>
__global__ __launch_bounds__(WAVES * 64)
void norm_bwd_held(BwdParams p)
{
    static_assert(VEC == 1 || VEC == 4 || (VEC == 8 && sizeof(T) == 2), "VEC");
    static_assert(WAVES % WPR == 0, "whole rows per workgroup");
    constexpr int RPB = WAVES / WPR;
    static_assert(RPB == 1 || RPB == 2 || RPB == 4 || RPB == 8 || RPB == 16, "row slots meet in a binary tree");
    constexpr int NG = (OP == OP_LN) ? 2 : 1;
    constexpr int CAP = 64 * WPR * Q;  // accesses per row
    using VT = vf<VEC>;
    using DT = vd<VEC>;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wr = wave % WPR;
    const int rib = wave / WPR;
    const int d = p.d;
    const int nvec = (int)((unsigned)d / VEC);
    const float inv_d = p.inv_d;

    // (sum g, sum g xhat) of each wave, double-buffered across steps so one
    // barrier per step suffices
    __shared__ float2 xch[2][RPB][WPR];
    // row slots' partial sums meeting pairwise
    __shared__ VT tree[RPB > 1 ? RPB / 2 : 1][RPB > 1 ? NG * CAP : 1];

    int kc[Q];
    bool okc[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int k = lane + 64 * (wr + WPR * q);
        okc[q] = k < nvec;
        kc[q] = k < nvec ? k : nvec - 1;
    }

    DT accg[Q], accb[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        accg[q] = DT(0.0);
        accb[q] = DT(0.0);
    }
    const bool want_pg = p.part != nullptr;
    // a lane keeps its columns for every row it visits, so gamma (or w) is
    // fetched once and held, not once per row
    VT gam[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) gam[q] = ldp<VEC>(p.p0 + VEC * kc[q]);

    const int64_t ngroups = (p.rows + RPB - 1) / RPB;
    // a row slot past the end (last step only) re-reads the last row and
    // stores nothing; loads stay unconditional at clamped addresses
    auto row_of = [&](int64_t rg) -> int64_t {
        const int64_t r = rg * RPB + rib;
        return r < p.rows ? r : p.rows - 1;
    };
    // x and dy of the step's row.  With one wave per row and at most 16
    // values per lane (PF), also the next step's: its loads are in flight
    // while this row is reduced and written (4% on [4096,768]; wider rows
    // gained nothing and would spill with the second copy).
    constexpr bool PF = WPR == 1 && VEC * Q <= 16;
    VT xv[Q], dv[Q];
    auto load_row = [&](int64_t row, VT (&xa)[Q], VT (&da)[Q]) {
        const T *xr = static_cast<const T *>(p.x) + row * p.ldx;
        const T *dyr = static_cast<const T *>(p.dy) + row * p.lddy;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            xa[q] = ldv<T, VEC, true>(xr + VEC * kc[q]);
            da[q] = ldv<T, VEC, true>(dyr + VEC * kc[q]);
        }
    };
    if constexpr (PF) {
        if ((int64_t)blockIdx.x < ngroups) load_row(row_of(blockIdx.x), xv, dv);
    }
    int par = 0;
    for (int64_t rg = blockIdx.x; rg < ngroups; rg += gridDim.x) {
        const int64_t row_raw = rg * RPB + rib;
        const bool rv = row_raw < p.rows;
        const int64_t row = rv ? row_raw : p.rows - 1;
        T *dxr = static_cast<T *>(p.dx) + row * p.lddx;
        const float mu = (OP == OP_LN) ? p.mean[row] : 0.f;
        const float rs = p.rstd[row];
        VT xn[PF ? Q : 1], dn[PF ? Q : 1];
        if constexpr (PF) {
            const int64_t nrg = rg + gridDim.x;
            if (nrg < ngroups) load_row(row_of(nrg), xn, dn);
        } else {
            load_row(row, xv, dv);
        }

        // xhat and g are formed twice (here for the sums, below for the
        // outputs) rather than held: only x and dy stay in registers
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const VT xh = (xv[q] - mu) * rs;
            const VT g = dv[q] * gam[q];
            s1 += okc[q] ? hsum(g) : 0.f;
            s2 += okc[q] ? hsum(g * xh) : 0.f;
        }
        float S1 = (OP == OP_LN) ? group_sum<64>(s1) : 0.f;
        float S2 = group_sum<64>(s2);
        if constexpr (WPR > 1) {
            if (lane == 0) xch[par][rib][wr] = make_float2(S1, S2);
            __syncthreads();
            S1 = 0.f;
            S2 = 0.f;
#pragma unroll
            for (int w = 0; w < WPR; ++w) {
                const float2 e = xch[par][rib][w];
                S1 += e.x;
                S2 += e.y;
            }
            par ^= 1;
        }
        const float m1 = S1 * inv_d, m2 = S2 * inv_d;

#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const VT xh = (xv[q] - mu) * rs;
            const VT g = dv[q] * gam[q];
            VT o;
            if constexpr (OP == OP_LN) o = rs * (g - m1 - xh * m2);
            else o = rs * (g - xh * m2);
            if (rv && okc[q]) stv<T, VEC, true>(dxr + VEC * kc[q], o);
            if (want_pg && rv && okc[q]) {
                accg[q] += widen64<VEC>(dv[q] * xh);
                if constexpr (OP == OP_LN) accb[q] += widen64<VEC>(dv[q]);
            }
        }
        if constexpr (PF) {
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                xv[q] = xn[q];
                dv[q] = dn[q];
            }
        }
    }
    if (!want_pg) return;

    // the workgroup's row slots meet pairwise (float32), slot 0 writes
    VT pg[Q], pb[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        pg[q] = narrow32<VEC>(accg[q]);
        pb[q] = narrow32<VEC>(accb[q]);
    }
    if constexpr (RPB > 1) {
        const int slot = wr * 64 + lane;
#pragma unroll
        for (int half = RPB / 2; half >= 1; half /= 2) {
            if (rib >= half && rib < 2 * half) {
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    tree[rib - half][slot + 64 * WPR * q] = pg[q];
                    if constexpr (NG == 2) tree[rib - half][CAP + slot + 64 * WPR * q] = pb[q];
                }
            }
            __syncthreads();
            if (rib < half) {
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    pg[q] += tree[rib][slot + 64 * WPR * q];
                    if constexpr (NG == 2) pb[q] += tree[rib][CAP + slot + 64 * WPR * q];
                }
            }
            __syncthreads();
        }
    }
    if (rib == 0) {
        float *pr = p.part + (int64_t)blockIdx.x * NG * p.dpad;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            if (!okc[q]) continue;
            stp<VEC>(pr + VEC * kc[q], pg[q]);
            if constexpr (NG == 2) stp<VEC>(pr + p.dpad + VEC * kc[q], pb[q]);
        }
    }
}

// ---------------------------------------------------------------------------
// Sum of the partial rows: out_g[j] = sum_b part[b][g][j] in float64, in a
// fixed order.  A workgroup covers 16 columns: 4 column quads by 64 slices of
// the partial rows (slice s takes rows s, s + 64, ...; with at most 256
// partial rows a lane issues at most 4 loads, all before any add), then the
// slices meet in a fixed binary tree in LDS.  Memory-latency bound: many
// small workgroups.
template <int NG>
__global__ __launch_bounds__(256)
void norm_bwd_reduce(const float *part, int64_t nblk, int32_t d, int32_t dpad, float *out0, float *out1)
{
    constexpr int SL = 64, CQ = 4, U = 4;
    const int cq = threadIdx.x % CQ;
    const int sl = threadIdx.x / CQ;
    const int g = blockIdx.y;
    const int col = (blockIdx.x * CQ + cq) * 4;
    __shared__ d4 red[SL][CQ];
    d4 acc = d4(0.0);
    if (col < dpad) {
        const float *base = part + (int64_t)g * dpad + col;
        for (int64_t b0 = sl; b0 < nblk; b0 += (int64_t)SL * U) {
            f4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t b = b0 + (int64_t)SL * u;
                v[u] = b < nblk ? ld4<false>(base + b * NG * dpad) : f4(0.f);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) acc += __builtin_convertvector(v[u], d4);
        }
    }
    red[sl][cq] = acc;
    __syncthreads();
#pragma unroll
    for (int half = SL / 2; half >= 1; half /= 2) {
        if (sl < half) red[sl][cq] += red[sl + half][cq];
        __syncthreads();
    }
    if (sl == 0 && col < d) {
        const d4 t = red[0][cq];
        float *out = g == 0 ? out0 : out1;
        if (out) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (col + i < d) out[col + i] = (float)t[i];
        }
    }
}

// ---------------------------------------------------------------------------
// Streamed rows, step 1: per row, stats = (mean_j g, mean_j g xhat); one
// workgroup of WAVES waves per row (grid-stride), single-element accesses.
// A lane adds its d / (64 WAVES) terms in float64 so that the rounding of
// the means stays that of a short sum however wide the row.
template <typename T, int OP, int WAVES>
__global__ __launch_bounds__(WAVES * 64)
void norm_bwd_rowstats(BwdParams p)
{
    __shared__ float red[2][WAVES];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    int slot = 0;
    for (int64_t row = blockIdx.x; row < p.rows; row += gridDim.x) {
        const T *xr = static_cast<const T *>(p.x) + row * p.ldx;
        const T *dyr = static_cast<const T *>(p.dy) + row * p.lddy;
        const float mu = (OP == OP_LN) ? p.mean[row] : 0.f;
        const float rs = p.rstd[row];
        double s1 = 0.0, s2 = 0.0;
        for (int j = tid; j < p.d; j += WAVES * 64) {
            const float xh = (lde<T, false>(xr + j) - mu) * rs;
            const float g = lde<T, false>(dyr + j) * p.p0[j];
            s1 += (double)g;
            s2 += (double)(g * xh);
        }
        const float S1 = (OP == OP_LN) ? block_sum<WAVES>((float)s1, red, slot, wave, lane) : 0.f;
        const float S2 = block_sum<WAVES>((float)s2, red, slot, wave, lane);
        if (tid == 0) p.stats[row] = make_float2(S1 * p.inv_d, S2 * p.inv_d);
    }
}

// Streamed rows, step 2: workgroup (blockIdx.x, blockIdx.y) covers column
// chunk x (WAVES * 64 * U elements, single-element accesses) of the rows of
// row block y; it writes dx there and the block's partial sums of those
// columns into partial row y.
template <typename T, int OP, int WAVES, int U>
__global__ __launch_bounds__(WAVES * 64)
void norm_bwd_chunks(BwdParams p, int64_t rows_per_block)
{
    constexpr int NG = (OP == OP_LN) ? 2 : 1;
    constexpr int NT = WAVES * 64;
    const int tid = threadIdx.x;
    const int64_t c0 = (int64_t)blockIdx.x * NT * U;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < p.rows ? r0 + rows_per_block : p.rows;
    double accg[U], accb[U];
    float gm[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t j = c0 + tid + NT * u;
        ok[u] = j < p.d;
        gm[u] = ok[u] ? p.p0[j] : 0.f;
        accg[u] = 0.0;
        accb[u] = 0.0;
    }
    for (int64_t row = r0; row < r1; ++row) {
        const T *xr = static_cast<const T *>(p.x) + row * p.ldx;
        const T *dyr = static_cast<const T *>(p.dy) + row * p.lddy;
        T *dxr = static_cast<T *>(p.dx) + row * p.lddx;
        const float mu = (OP == OP_LN) ? p.mean[row] : 0.f;
        const float rs = p.rstd[row];
        const float2 st = p.stats[row];
        float xv[U], dv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = c0 + tid + NT * u;
            xv[u] = ok[u] ? lde<T, false>(xr + j) : 0.f;
            dv[u] = ok[u] ? lde<T, false>(dyr + j) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!ok[u]) continue;
            const int64_t j = c0 + tid + NT * u;
            const float xh = (xv[u] - mu) * rs;
            const float g = dv[u] * gm[u];
            const float o = (OP == OP_LN) ? rs * (g - st.x - xh * st.y) : rs * (g - xh * st.y);
            ste<T, false>(dxr + j, o);
            accg[u] += (double)(dv[u] * xh);
            accb[u] += (double)dv[u];
        }
    }
    if (p.part == nullptr) return;
    float *pr = p.part + (int64_t)blockIdx.y * NG * p.dpad;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        const int64_t j = c0 + tid + NT * u;
        pr[j] = (float)accg[u];
        if constexpr (NG == 2) pr[p.dpad + j] = (float)accb[u];
    }
}

}  // namespace minorm
