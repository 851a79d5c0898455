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
// registers; at the end the row slots of the workgroup stage their sums in
// LDS and the workgroup writes one float32 partial row; a second kernel sums
// the partial rows in float64 in a fixed order (deterministic results).
// Rows of several waves load each step's inputs while the previous step
// runs (two input sets; see norm_bwd_held).
//
// Accumulation contract: every term (g, g xhat, dy xhat, dy) is formed in
// float32 from the float32 inputs.  A row's two sums add the terms in
// groups of at most eight, pairwise, in float32 and carry everything from
// there in float64 (lanes, waves); each mean is rounded once to float32.
// A column sum is carried in float64 per lane, rounded once to float32 per
// row slot, the slots of a workgroup added in float64 and rounded once to
// the workgroup's partial row, and the partial rows added in float64 and
// rounded once.  The error of the results is then bounded by a few float32
// roundings of each term, however the rows and columns are split among
// lanes, waves and workgroups.
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

// float64 cross-lane moves: the two 32-bit halves move separately.  With
// every row and bank enabled the destination's old value is not used; a
// partial row mask keeps zero in the rows not written.
typedef int i2 __attribute__((ext_vector_type(2)));
template <int CTRL>
__device__ __forceinline__ double dpp64(double v) {
    const i2 b = __builtin_bit_cast(i2, v);
    i2 r;
    r.x = __builtin_amdgcn_mov_dpp(b.x, CTRL, 0xF, 0xF, false);
    r.y = __builtin_amdgcn_mov_dpp(b.y, CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, r);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp64_rows(double v) {
    const i2 b = __builtin_bit_cast(i2, v);
    i2 r;
    r.x = __builtin_amdgcn_update_dpp(0, b.x, CTRL, ROWS, 0xF, false);
    r.y = __builtin_amdgcn_update_dpp(0, b.y, CTRL, ROWS, 0xF, false);
    return __builtin_bit_cast(double, r);
}
__device__ __forceinline__ double readlane64(double v, int lane) {
    const i2 b = __builtin_bit_cast(i2, v);
    i2 r;
    r.x = __builtin_amdgcn_readlane(b.x, lane);
    r.y = __builtin_amdgcn_readlane(b.y, lane);
    return __builtin_bit_cast(double, r);
}

// Sum over the 64 lanes of a wave in float64, in a fixed order: butterflies
// within each 16-lane row, then row_bcast:15 adds row 0's sum into row 1 and
// row 2's into row 3, row_bcast:31 adds rows 0-1 into rows 2-3; lane 63 ends
// with the total, read into scalars (a wave-uniform result).
__device__ __forceinline__ double wave_sum64(double v) {
    v += dpp64<0xB1>(v);            // lane ^ 1
    v += dpp64<0x4E>(v);            // lane ^ 2
    v += dpp64<0x141>(v);           // the other quad of each 8 lanes
    v += dpp64<0x140>(v);           // the other half of each 16-lane row
    v += dpp64_rows<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp64_rows<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return readlane64(v, 63);
}

// Pairwise float32 sum of N values (N <= 8: at most three roundings per value)
template <int N>
__device__ __forceinline__ float pair_sum(const float *a) {
    if constexpr (N == 1) return a[0];
    else return pair_sum<N / 2>(a) + pair_sum<N - N / 2>(a + N / 2);
}

// Sum over a workgroup's WAVES waves in float64: wave sums, one LDS exchange
// (double-buffered by slot, so one barrier per call), waves added in order.
template <int WAVES>
__device__ __forceinline__ double block_sum64(double v, double (*red)[WAVES], int &slot, int wave, int lane) {
    v = wave_sum64(v);
    if (lane == 0) red[slot][wave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) t += red[slot][w];
    slot ^= 1;
    return t;
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
    double inv_d;         // 1 / d
};

// ---------------------------------------------------------------------------
// One row slot's inputs for one step of the pipelined loop below: x and dy as
// loaded (16-byte accesses, or single elements, not yet widened) and the
// row's statistics.
template <typename T, int VEC, int Q>
struct RowIn {
    using R = std::conditional_t<VEC == 1, uint32_t, u4>;
    R x[Q], dy[Q];
    float mu, rs;
};

// what one access loaded, widened to float32
template <typename T, int VEC>
__device__ __forceinline__ vf<VEC> widen_raw(std::conditional_t<VEC == 1, uint32_t, u4> r) {
    if constexpr (VEC == 1) {
        if constexpr (std::is_same_v<T, float>) return __builtin_bit_cast(float, r);
        else return (float)__builtin_bit_cast(T, (uint16_t)r);
    } else if constexpr (std::is_same_v<T, float>) {
        static_assert(VEC == 4, "four float32 per access");
        return __builtin_bit_cast(f4, r);
    } else {
        static_assert(VEC == 8 && sizeof(T) == 2, "eight 16-bit elements per access");
        typedef T t8 __attribute__((ext_vector_type(8)));
        return __builtin_convertvector(__builtin_bit_cast(t8, r), f8);
    }
}

// ---------------------------------------------------------------------------
// Held rows.
//   T      storage type of dy, x, dx
//   OP     OP_LN or OP_RMS
//   VEC    elements per access: 4 (float32) / 8 (16-bit) with aligned rows, or 1
//   WPR    waves per row; WAVES / WPR rows per workgroup per step (1, 2, 4, 8)
//   Q      accesses held per lane; capacity VEC * 64 * WPR * Q elements
// Lane li of wave rank wr holds access k = li + 64 * (wr + WPR * q) of every
// row its row slot visits.
//
// Rows of several waves with at most 16 values per lane run a pipelined
// loop: two input sets alternate, and a step's loads (raw buffer loads over
// the row, so a prefetch past the last row moves no data) are issued before
// the previous step's sums, which wait only for their own set.  The waves of
// a row meet at a barrier every step, so without the second set a
// workgroup's loads and its arithmetic never overlap (BF16 LayerNorm
// [32768,8192] 320 against 273 us, [8192,3072] 61 against 56).  16-bit rows
// of one wave take it too (BF16 LayerNorm [8192,512] 13.1 against 11.3 us,
// [65536,768] 63.8 against 58.3, [4096,768] 2-3%).  Float32 rows of one
// wave keep the loop that prefetches the next row into a copy (with the
// alternating sets [4096,768] ran 4% and [65536,768] 6% slower).
template <typename T, int OP, int VEC, int WPR, int Q, int WAVES>
__global__ __launch_bounds__(WAVES * 64)
void norm_bwd_held(BwdParams p)
{
    static_assert(VEC == 1 || VEC == 4 || (VEC == 8 && sizeof(T) == 2), "VEC");
    static_assert(WAVES % WPR == 0, "whole rows per workgroup");
    constexpr int RPB = WAVES / WPR;
    static_assert(RPB == 1 || RPB == 2 || RPB == 4 || RPB == 8 || RPB == 16, "1, 2, 4, 8 or 16 row slots");
    constexpr int NG = (OP == OP_LN) ? 2 : 1;
    using VT = vf<VEC>;
    using DT = vd<VEC>;
    constexpr bool PIPE = VEC * Q <= 16 && (WPR > 1 || VEC == 8);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wr = wave % WPR;
    const int rib = wave / WPR;
    const int d = p.d;
    const int nvec = (int)((unsigned)d / VEC);
    const double inv_d = p.inv_d;

    // (sum g, sum g xhat) of each wave, double-buffered across steps so one
    // barrier per step suffices
    __shared__ double xch[2][RPB][WPR][2];
    // the row slots' partial column sums (float32), for the workgroup's sum
    constexpr int TW = 64 * WPR;   // lanes per row slot
    constexpr int NV = TW * Q;     // accesses per partial row
    __shared__ VT stage[RPB > 1 ? RPB : 1][RPB > 1 ? NG : 1][RPB > 1 ? NV : 1];

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
    int par = 0;
    // One step of row group rg: the row's two sums, dx, and the terms of the
    // column sums.  A row slot past the end (last step only) stores nothing.
    auto step = [&](int64_t rg, const VT (&xv)[Q], const VT (&dv)[Q], float mu, float rs) {
        const int64_t row_raw = rg * RPB + rib;
        const bool rv = row_raw < p.rows;
        const int64_t row = rv ? row_raw : p.rows - 1;
        T *dxr = static_cast<T *>(p.dx) + row * p.lddx;

        // xhat and g: with at most 16 values per lane formed once and held
        // until the outputs (BF16 LayerNorm [32768,8192] 2.4% faster); wider
        // lanes form them again for the outputs, keeping only x and dy.  The
        // terms of a group of eight (one 16-bit access, two float32 ones,
        // eight single elements) are added pairwise in float32, the groups in
        // float64.
        constexpr bool HOLD = VEC * Q <= 16;
        VT xhs[HOLD ? Q : 1], gs[HOLD ? Q : 1];
        if constexpr (HOLD) {
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                xhs[q] = (xv[q] - mu) * rs;
                gs[q] = dv[q] * gam[q];
            }
        }
        auto xh_of = [&](int q) -> VT {
            if constexpr (HOLD) return xhs[q];
            else return (xv[q] - mu) * rs;
        };
        auto g_of = [&](int q) -> VT {
            if constexpr (HOLD) return gs[q];
            else return dv[q] * gam[q];
        };
        double s1 = 0.0, s2 = 0.0;
        if constexpr (VEC == 8 || Q == 1) {
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const VT xh = xh_of(q);
                const VT g = g_of(q);
                if (okc[q]) {
                    if (OP == OP_LN) s1 += (double)hsum(g);
                    s2 += (double)hsum(g * xh);
                }
            }
        } else {
            // access q0 + j of a group lies past the row's end when q0 does
            constexpr int GA = 8 / VEC;  // accesses per group
#pragma unroll
            for (int q0 = 0; q0 < Q; q0 += GA) {
                if (!okc[q0]) continue;
                float t1[GA], t2[GA];
#pragma unroll
                for (int j = 0; j < GA; ++j) {
                    const int q = q0 + j;
                    t1[j] = 0.f;
                    t2[j] = 0.f;
                    if (q < Q) {
                        const VT xh = xh_of(q);
                        const VT g = g_of(q);
                        t1[j] = okc[q] ? hsum(g) : 0.f;
                        t2[j] = okc[q] ? hsum(g * xh) : 0.f;
                    }
                }
                if (OP == OP_LN) s1 += (double)pair_sum<GA>(t1);
                s2 += (double)pair_sum<GA>(t2);
            }
        }
        double S1 = (OP == OP_LN) ? wave_sum64(s1) : 0.0;
        double S2 = wave_sum64(s2);
        if constexpr (WPR > 1) {
            if (lane == 0) {
                xch[par][rib][wr][0] = S1;
                xch[par][rib][wr][1] = S2;
            }
            __syncthreads();
            S1 = 0.0;
            S2 = 0.0;
#pragma unroll
            for (int w = 0; w < WPR; ++w) {
                S1 += xch[par][rib][w][0];
                S2 += xch[par][rib][w][1];
            }
            par ^= 1;
        }
        const float m1 = (float)(S1 * inv_d), m2 = (float)(S2 * inv_d);

#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const VT xh = xh_of(q);
            const VT g = g_of(q);
            VT o;
            if constexpr (OP == OP_LN) o = rs * (g - m1 - xh * m2);
            else o = rs * (g - xh * m2);
            if (rv && okc[q]) stv<T, VEC, true>(dxr + VEC * kc[q], o);
            if (want_pg && rv && okc[q]) {
                accg[q] += widen64<VEC>(dv[q] * xh);
                if constexpr (OP == OP_LN) accb[q] += widen64<VEC>(dv[q]);
            }
        }
    };

    if constexpr (PIPE) {
        using In = RowIn<T, VEC, Q>;
        constexpr uint32_t ES = sizeof(T);
        const uint32_t row_bytes = (uint32_t)d * ES;
        uint32_t voff[Q];   // past the row's end the range check reads zero
#pragma unroll
        for (int q = 0; q < Q; ++q) voff[q] = (uint32_t)(lane + 64 * (wr + WPR * q)) * (ES * VEC);
        // x, dy and the statistics of row group rg, each through a raw buffer
        // over exactly what it reads: empty for a row past the end, whose
        // loads then read zero and move no data
        auto load = [&](int64_t rg, In &S) {
            const int64_t r = rg * RPB + rib;
            const bool ok = r < p.rows;
            const int64_t rc = ok ? r : p.rows - 1;
            const auto bx = row_buffer(static_cast<const T *>(p.x) + rc * p.ldx, ok ? row_bytes : 0u);
            const auto bdy = row_buffer(static_cast<const T *>(p.dy) + rc * p.lddy, ok ? row_bytes : 0u);
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                if constexpr (VEC > 1) {
                    S.x[q] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(bx, (int)voff[q], 0, 2));
                    S.dy[q] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(bdy, (int)voff[q], 0, 2));
                } else if constexpr (ES == 4) {
                    S.x[q] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(bx, (int)voff[q], 0, 2);
                    S.dy[q] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(bdy, (int)voff[q], 0, 2);
                } else {
                    S.x[q] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(bx, (int)voff[q], 0, 2);
                    S.dy[q] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(bdy, (int)voff[q], 0, 2);
                }
            }
            S.mu = 0.f;
            if constexpr (OP == OP_LN)
                S.mu = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(row_buffer(p.mean + rc, ok ? 4u : 0u), 0, 0, 0));
            S.rs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(row_buffer(p.rstd + rc, ok ? 4u : 0u), 0, 0, 0));
        };
        // A set's values are used only after this point, which the loads
        // issued before it may not pass: they stay in flight during the step.
        auto run = [&](int64_t rg, In &S) {
#pragma unroll
            for (int q = 0; q < Q; ++q) asm volatile("" : "+v"(S.x[q]), "+v"(S.dy[q])::"memory");
            asm volatile("" : "+v"(S.mu), "+v"(S.rs)::"memory");
            VT xv[Q], dv[Q];
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                xv[q] = widen_raw<T, VEC>(S.x[q]);
                dv[q] = widen_raw<T, VEC>(S.dy[q]);
            }
            step(rg, xv, dv, S.mu, S.rs);
        };
        const int64_t G = gridDim.x;
        int64_t rg = blockIdx.x;
        if (rg < ngroups) {
            In A, B;
            load(rg, A);
            for (;;) {
                load(rg + G, B);
                run(rg, A);
                if (rg + G >= ngroups) break;
                load(rg + 2 * G, A);
                run(rg + G, B);
                rg += 2 * G;
                if (rg >= ngroups) break;
            }
        }
    } else {
        // a row slot past the end re-reads the last row; loads stay
        // unconditional at clamped addresses
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
        for (int64_t rg = blockIdx.x; rg < ngroups; rg += gridDim.x) {
            const int64_t row = row_of(rg);
            const float mu = (OP == OP_LN) ? p.mean[row] : 0.f;
            const float rs = p.rstd[row];
            VT xn[PF ? Q : 1], dn[PF ? Q : 1];
            if constexpr (PF) {
                const int64_t nrg = rg + gridDim.x;
                if (nrg < ngroups) load_row(row_of(nrg), xn, dn);
            } else {
                load_row(row, xv, dv);
            }
            step(rg, xv, dv, mu, rs);
            if constexpr (PF) {
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    xv[q] = xn[q];
                    dv[q] = dn[q];
                }
            }
        }
    }
    if (!want_pg) return;

    float *pr = p.part + (int64_t)blockIdx.x * NG * p.dpad;
    if constexpr (RPB == 1) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            if (!okc[q]) continue;
            stp<VEC>(pr + VEC * kc[q], narrow32<VEC>(accg[q]));
            if constexpr (NG == 2) stp<VEC>(pr + p.dpad + VEC * kc[q], narrow32<VEC>(accb[q]));
        }
    } else {
        // each row slot rounds its sums once and stages them; then every
        // thread takes some accesses of the partial row and adds the slots'
        // values in float64, in slot order, rounding once
        const int sl = wr * 64 + lane;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            stage[rib][0][sl + TW * q] = narrow32<VEC>(accg[q]);
            if constexpr (NG == 2) stage[rib][1][sl + TW * q] = narrow32<VEC>(accb[q]);
        }
        __syncthreads();
        for (int i = tid; i < NG * NV; i += WAVES * 64) {
            const int gi = i / NV, k = i - gi * NV;
            if (k >= nvec) continue;
            DT t = DT(0.0);
#pragma unroll
            for (int r = 0; r < RPB; ++r) t += widen64<VEC>(stage[r][gi][k]);
            stp<VEC>(pr + gi * p.dpad + VEC * k, narrow32<VEC>(t));
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
// workgroup of WAVES waves per row (grid-stride).  VEC elements per access
// (16-byte accesses on aligned rows, else single elements), U accesses per
// lane in flight.  The terms of an access are added pairwise in float32 (a
// group of at most eight), the groups in float64 (lanes, waves, the
// workgroup), and each mean is rounded once.
template <typename T, int OP, int VEC, int WAVES, int U>
__global__ __launch_bounds__(WAVES * 64)
void norm_bwd_rowstats(BwdParams p)
{
    using VT = vf<VEC>;
    constexpr int NT = WAVES * 64;
    __shared__ double red[2][WAVES];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int nvec = (int)((unsigned)p.d / VEC);
    int slot = 0;
    for (int64_t row = blockIdx.x; row < p.rows; row += gridDim.x) {
        const T *xr = static_cast<const T *>(p.x) + row * p.ldx;
        const T *dyr = static_cast<const T *>(p.dy) + row * p.lddy;
        const float mu = (OP == OP_LN) ? p.mean[row] : 0.f;
        const float rs = p.rstd[row];
        double s1 = 0.0, s2 = 0.0;
        for (int k0 = tid; k0 < nvec; k0 += NT * U) {
            VT xv[U], dv[U], gv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = k0 + NT * u;
                const int kc = k < nvec ? k : nvec - 1;
                xv[u] = ldv<T, VEC, true>(xr + VEC * kc);
                dv[u] = ldv<T, VEC, true>(dyr + VEC * kc);
                gv[u] = ldp<VEC>(p.p0 + VEC * kc);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (k0 + NT * u >= nvec) continue;
                const VT xh = (xv[u] - mu) * rs;
                const VT g = dv[u] * gv[u];
                if (OP == OP_LN) s1 += (double)hsum(g);
                s2 += (double)hsum(g * xh);
            }
        }
        const double S1 = (OP == OP_LN) ? block_sum64<WAVES>(s1, red, slot, wave, lane) : 0.0;
        const double S2 = block_sum64<WAVES>(s2, red, slot, wave, lane);
        if (tid == 0) p.stats[row] = make_float2((float)(S1 * p.inv_d), (float)(S2 * p.inv_d));
    }
}

// Streamed rows, step 2: workgroup (blockIdx.x, blockIdx.y) covers column
// chunk x (WAVES * 64 * U accesses of VEC elements) of the rows of row block
// y; it writes dx there and the block's partial sums of those columns into
// partial row y.  The next row's x and dy are loaded while a row is written.
template <typename T, int OP, int VEC, int WAVES, int U>
__global__ __launch_bounds__(WAVES * 64)
void norm_bwd_chunks(BwdParams p, int64_t rows_per_block)
{
    using VT = vf<VEC>;
    using DT = vd<VEC>;
    constexpr int NG = (OP == OP_LN) ? 2 : 1;
    constexpr int NT = WAVES * 64;
    const int tid = threadIdx.x;
    const int nvec = (int)((unsigned)p.d / VEC);
    const int64_t k0 = (int64_t)blockIdx.x * NT * U + tid;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < p.rows ? r0 + rows_per_block : p.rows;
    DT accg[U], accb[U];
    VT gm[U];
    int kc[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t k = k0 + NT * u;
        ok[u] = k < nvec;
        kc[u] = ok[u] ? (int)k : nvec - 1;
        gm[u] = ldp<VEC>(p.p0 + VEC * kc[u]);
        accg[u] = DT(0.0);
        accb[u] = DT(0.0);
    }
    VT xv[U], dv[U];
    auto load_row = [&](int64_t row, VT (&xa)[U], VT (&da)[U]) {
        const T *xr = static_cast<const T *>(p.x) + row * p.ldx;
        const T *dyr = static_cast<const T *>(p.dy) + row * p.lddy;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            xa[u] = ldv<T, VEC, true>(xr + VEC * kc[u]);
            da[u] = ldv<T, VEC, true>(dyr + VEC * kc[u]);
        }
    };
    if (r0 < r1) load_row(r0, xv, dv);
    for (int64_t row = r0; row < r1; ++row) {
        T *dxr = static_cast<T *>(p.dx) + row * p.lddx;
        const float mu = (OP == OP_LN) ? p.mean[row] : 0.f;
        const float rs = p.rstd[row];
        const float2 st = p.stats[row];
        VT xn[U], dn[U];
        if (row + 1 < r1) load_row(row + 1, xn, dn);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!ok[u]) continue;
            const VT xh = (xv[u] - mu) * rs;
            const VT g = dv[u] * gm[u];
            VT o;
            if constexpr (OP == OP_LN) o = rs * (g - st.x - xh * st.y);
            else o = rs * (g - xh * st.y);
            stv<T, VEC, true>(dxr + VEC * kc[u], o);
            accg[u] += widen64<VEC>(dv[u] * xh);
            if constexpr (OP == OP_LN) accb[u] += widen64<VEC>(dv[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            xv[u] = xn[u];
            dv[u] = dn[u];
        }
    }
    if (p.part == nullptr) return;
    float *pr = p.part + (int64_t)blockIdx.y * NG * p.dpad;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        stp<VEC>(pr + VEC * kc[u], narrow32<VEC>(accg[u]));
        if constexpr (NG == 2) stp<VEC>(pr + p.dpad + VEC * kc[u], narrow32<VEC>(accb[u]));
    }
}

}  // namespace minorm
