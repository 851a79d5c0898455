// norm_kernels.hpp — gfx950 device code for forward LayerNorm / RMSNorm.
//
// The shape follows what "Field note 004: The load in flight, and the shape
// Triton uses" (section "The layer norm was rewritten in the shape Triton
// uses") found decisive: one pass over x, the row held in registers from load
// to store, partial sums meeting once.  On CDNA4 that becomes:
//
//  * A row is owned by a 16/32/64-lane group of one wave64, or by W waves of a
//    workgroup.  Each lane issues all of its 128-bit loads
//    (global_load_dwordx4) before using any, keeping Q of them in VGPRs.
//  * Statistics reduce inside the wave with DPP butterflies
//    (quad_perm, row_half_mirror, row_mirror), then ds_swizzle or
//    v_readlane across 16-lane rows: no LDS, no barrier.  When W > 1 waves
//    share a row, each wave reduces its own (mean, centered M2) and the waves
//    meet once in LDS behind one barrier, merged with the pairwise formula of
//    Chan, Golub and LeVeque — the counterpart of the single exchange of
//    "How the kernel time fell, step by step" (section "The layer norm was
//    short of resident threads"), without its one-pass sum of squares.
//  * rstd is v_rsq_f32, the one-instruction reciprocal root; gamma/beta are
//    read once per row group and y leaves the same registers in 128-bit stores.
//  * Rows may be stored as float32, binary16 or bfloat16 (template T): an
//    access always carries four elements (16 or 8 bytes), widened exactly to
//    float32 in registers; statistics, parameters and arithmetic stay float32
//    and each output is rounded once to T (v_cvt_pk_f16_f32 /
//    v_cvt_pk_bf16_f32, round to nearest even).  Each row tensor has its own
//    row stride in elements.
//
// Every lane of a wave executes every cross-lane step (lanes with nothing to
// hold contribute zeros), so DPP sources are always active lanes and every
// workgroup reaches every barrier the same number of times.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace minorm {

enum : int { OP_LN = 0, OP_RMS = 1 };

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f8 __attribute__((ext_vector_type(8)));
typedef unsigned int u2 __attribute__((ext_vector_type(2)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

// float32 registers holding VEC elements (1, 4 or 8)
template <int VEC> struct VecOf;
template <> struct VecOf<1> { using type = float; };
template <> struct VecOf<4> { using type = f4; };
template <> struct VecOf<8> { using type = f8; };
template <int VEC> using vf = typename VecOf<VEC>::type;

// Kernel arguments (one struct, passed by value).  Row tensors hold elements
// of the kernel's storage type T; ld* are their row strides in elements.
struct NormParams {
    const void *x;
    const float *p0;   // gamma (LayerNorm) or w (RMSNorm)
    const float *p1;   // beta (LayerNorm); unused by RMSNorm
    void *y;
    float *mean;       // LayerNorm only; may be null
    float *rstd;       // may be null
    const void *r;     // residual added to x before the norm (RES kernels)
    void *h;           // x + r written out (RES kernels); may be null
    int64_t rows;      // rows of this launch
    int64_t ldx, ldr, ldy, ldh;
    int32_t d;
    float eps;
    float inv_d;       // 1/d rounded to float32
    int32_t peel_align;  // peeled rows: the body starts on a multiple of this
                         // many elements (16 bytes', or 128 bytes' when every
                         // row tensor shares its phase within a cache line)
};

// ---------------------------------------------------------------------------
// cross-lane sums

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float readlane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over aligned groups of G lanes (G = 16, 32 or 64).  Every lane of a
// group ends with the same bits: each step adds a partner's value, and the
// two partners add the same pair (IEEE addition commutes).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(G == 16 || G == 32 || G == 64, "group of 16, 32 or 64 lanes");
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
    v += dpp<0x141>(v);  // row_half_mirror: the other quad of each 8 lanes
    v += dpp<0x140>(v);  // row_mirror: the other half of each 16-lane row
    if constexpr (G == 32) {
        // ds_swizzle bit mode, and_mask 0x1f, xor_mask 0x10: lane ^ 16 within 32
        v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
    } else if constexpr (G == 64) {
        // the four 16-lane row sums, read into scalars: a wave-uniform result
        const float r0 = readlane(v, 0), r1 = readlane(v, 16);
        const float r2 = readlane(v, 32), r3 = readlane(v, 48);
        v = (r0 + r1) + (r2 + r3);
    }
    return v;
}

// ---------------------------------------------------------------------------
// memory helpers

template <bool NT>
__device__ __forceinline__ f4 ld4(const float *p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p));
    else return *reinterpret_cast<const f4 *>(p);
}

template <bool NT>
__device__ __forceinline__ float ld1(const float *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT>
__device__ __forceinline__ void st4(float *p, f4 v) {
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<f4 *>(p));
    else *reinterpret_cast<f4 *>(p) = v;
}

template <bool NT>
__device__ __forceinline__ void st1(float *p, float v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Storage-typed access: four elements (ldq/stq) or one (lde/ste) of T,
// widened to / rounded from float32.  float32 goes through the helpers above;
// a 16-bit quad is one 64-bit access.
template <typename T, bool NT>
__device__ __forceinline__ f4 ldq(const T *p) {
    if constexpr (std::is_same_v<T, float>) {
        return ld4<NT>(p);
    } else {
        typedef T t4 __attribute__((ext_vector_type(4)));
        u2 raw;
        if constexpr (NT) raw = __builtin_nontemporal_load(reinterpret_cast<const u2 *>(p));
        else raw = *reinterpret_cast<const u2 *>(p);
        return __builtin_convertvector(__builtin_bit_cast(t4, raw), f4);
    }
}

template <typename T, bool NT>
__device__ __forceinline__ float lde(const T *p) {
    if constexpr (std::is_same_v<T, float>) {
        return ld1<NT>(p);
    } else {
        unsigned short raw;
        if constexpr (NT) raw = __builtin_nontemporal_load(reinterpret_cast<const unsigned short *>(p));
        else raw = *reinterpret_cast<const unsigned short *>(p);
        return (float)__builtin_bit_cast(T, raw);
    }
}

template <typename T, bool NT>
__device__ __forceinline__ void stq(T *p, f4 v) {
    if constexpr (std::is_same_v<T, float>) {
        st4<NT>(p, v);
    } else {
        typedef T t4 __attribute__((ext_vector_type(4)));
        const u2 raw = __builtin_bit_cast(u2, __builtin_convertvector(v, t4));
        if constexpr (NT) __builtin_nontemporal_store(raw, reinterpret_cast<u2 *>(p));
        else *reinterpret_cast<u2 *>(p) = raw;
    }
}

template <typename T, bool NT>
__device__ __forceinline__ void ste(T *p, float v) {
    if constexpr (std::is_same_v<T, float>) {
        st1<NT>(p, v);
    } else {
        const unsigned short raw = __builtin_bit_cast(unsigned short, (T)v);
        if constexpr (NT) __builtin_nontemporal_store(raw, reinterpret_cast<unsigned short *>(p));
        else *reinterpret_cast<unsigned short *>(p) = raw;
    }
}

// An oct: eight 16-bit elements in one 128-bit access.
template <typename T, bool NT>
__device__ __forceinline__ f8 ldo(const T *p) {
    static_assert(sizeof(T) == 2, "octs are 16-bit elements");
    typedef T t8 __attribute__((ext_vector_type(8)));
    u4 raw;
    if constexpr (NT) raw = __builtin_nontemporal_load(reinterpret_cast<const u4 *>(p));
    else raw = *reinterpret_cast<const u4 *>(p);
    return __builtin_convertvector(__builtin_bit_cast(t8, raw), f8);
}

template <typename T, bool NT>
__device__ __forceinline__ void sto(T *p, f8 v) {
    static_assert(sizeof(T) == 2, "octs are 16-bit elements");
    typedef T t8 __attribute__((ext_vector_type(8)));
    const u4 raw = __builtin_bit_cast(u4, __builtin_convertvector(v, t8));
    if constexpr (NT) __builtin_nontemporal_store(raw, reinterpret_cast<u4 *>(p));
    else *reinterpret_cast<u4 *>(p) = raw;
}

// VEC consecutive elements of T (one access), widened to float32, and back
template <typename T, int VEC, bool NT>
__device__ __forceinline__ vf<VEC> ldv(const T *p) {
    if constexpr (VEC == 1) return lde<T, NT>(p);
    else if constexpr (VEC == 4) return ldq<T, NT>(p);
    else return ldo<T, NT>(p);
}

template <typename T, int VEC, bool NT>
__device__ __forceinline__ void stv(T *p, vf<VEC> v) {
    if constexpr (VEC == 1) ste<T, NT>(p, v);
    else if constexpr (VEC == 4) stq<T, NT>(p, v);
    else sto<T, NT>(p, v);
}

// VEC consecutive float32 parameters: 16-byte-aligned vector loads, or
// (unaligned, the peeled path) element by element
template <int VEC>
__device__ __forceinline__ vf<VEC> ldp(const float *p) {
    if constexpr (VEC == 1) return *p;
    else if constexpr (VEC == 4) return ld4<false>(p);
    else return __builtin_shufflevector(ld4<false>(p), ld4<false>(p + 4), 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int VEC>
__device__ __forceinline__ vf<VEC> ldp_scalar(const float *p) {
    vf<VEC> v;
    if constexpr (VEC == 1) {
        v = p[0];
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) v[i] = p[i];
    }
    return v;
}

// the value as stored in T (a rounding and an exact widening; identity for float)
template <typename T>
__device__ __forceinline__ f4 as_stored(f4 v) {
    if constexpr (std::is_same_v<T, float>) {
        return v;
    } else {
        typedef T t4 __attribute__((ext_vector_type(4)));
        return __builtin_convertvector(__builtin_convertvector(v, t4), f4);
    }
}
template <typename T>
__device__ __forceinline__ f8 as_stored(f8 v) {
    if constexpr (std::is_same_v<T, float>) {
        return v;
    } else {
        typedef T t8 __attribute__((ext_vector_type(8)));
        return __builtin_convertvector(__builtin_convertvector(v, t8), f8);
    }
}
template <typename T>
__device__ __forceinline__ float as_stored(float v) {
    if constexpr (std::is_same_v<T, float>) return v;
    else return (float)(T)v;
}

__device__ __forceinline__ float hsum(f4 v) { return (v.x + v.y) + (v.z + v.w); }
__device__ __forceinline__ float hsum(f8 v) { return hsum(v.lo) + hsum(v.hi); }
__device__ __forceinline__ float hsum(float v) { return v; }

__device__ __forceinline__ float csq(f4 v, float mu) {
    const f4 c = v - mu;
    return (c.x * c.x + c.y * c.y) + (c.z * c.z + c.w * c.w);
}
__device__ __forceinline__ float csq(float v, float mu) { const float c = v - mu; return c * c; }
__device__ __forceinline__ float csq(f8 v, float mu) { return csq(v.lo, mu) + csq(v.hi, mu); }

__device__ __forceinline__ float sq(f4 v) { return (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w); }
__device__ __forceinline__ float sq(float v) { return v * v; }
__device__ __forceinline__ float sq(f8 v) { return sq(v.lo) + sq(v.hi); }

__device__ __forceinline__ float rsq(float v) { return __builtin_amdgcn_rsqf(v); }

// an empty asm that takes v: the value must exist here (its load has
// returned), and nothing computed from it moves above this point
template <typename V>
__device__ __forceinline__ void keep(V &v) { asm volatile("" : "+v"(v)); }


// ---------------------------------------------------------------------------
// Held-row kernel.
//
//   T      storage type of the row tensors: float, _Float16 or __bf16
//   OP     OP_LN or OP_RMS
//   VEC    elements per lane access: 4 (a quad: 128-bit for float, 64-bit
//          for the 16-bit types), 8 (an oct: 128-bit, 16-bit types only) -
//          d % VEC == 0 and rows aligned to an access - or 1 (any d, any
//          element alignment)
//   PEEL   VEC > 1 only: per row, scalar head elements up to the row's first
//          p.peel_align boundary (16 bytes, or a 128-byte cache line), a
//          vector body, and a scalar tail; needs every row tensor in the
//          same phase modulo that boundary and d >= 128 (the body is never
//          empty); gamma/beta are read unaligned since their phase follows
//          the row's
//   LPR    lanes of one wave sharing a row (16, 32, 64); 64 / LPR rows per wave
//   WPR    waves sharing a row (LPR == 64 when WPR > 1)
//   Q      accesses held per lane; capacity = VEC * LPR * WPR * Q elements
//   WAVES  waves per workgroup
//   NTL/NTS  non-temporal x loads / y stores
//   RES    residual add fused before the norm: each held value is x + r
//          (a float32 add, rounded to T), written to h when h is given, and
//          the row is normalized from those stored sums
//   MRG    cross-wave merge: 0 every lane walks all WPR exchanged entries,
//          1 lane w takes entry w and two 16-lane sums finish the merge;
//          -1: 1 for 16 waves per row, else 0
//   PRE    where the output pass gets gamma/beta (or w): 0: global loads in
//          the output pass; 1: global loads issued while x is in flight;
//          2: staged once per workgroup in LDS at kernel start (aligned
//          16-byte path only), so each parameter crosses the CU's vector
//          memory path once per workgroup rather than once per row;
//          -1: 1 or 0 by the register budget
//
// Lane li of wave rank wr holds access k = li + LPR * (wr + WPR * q),
// q = 0..Q-1: consecutive lanes touch consecutive vectors (or elements), so
// each wave-wide access covers 64 vectors of one row contiguously (1 KiB on
// the vector paths).
template <typename T, int OP, int VEC, bool PEEL, int LPR, int WPR, int Q, int WAVES, bool NTL,
          bool NTS, int PRE = -1, int MRG = -1, bool RES = false>
__global__ __launch_bounds__(WAVES * 64)
void norm_held(NormParams p)
{
    static_assert(VEC == 1 || VEC == 4 || (VEC == 8 && sizeof(T) == 2), "VEC");
    static_assert(!PEEL || (VEC > 1 && LPR == 64), "PEEL needs vector accesses, full-wave rows");
    static_assert(LPR == 16 || LPR == 32 || LPR == 64, "LPR");
    static_assert(WPR == 1 || LPR == 64, "multi-wave rows use full waves");
    static_assert(WAVES % WPR == 0, "whole rows per workgroup");
    static_assert(WPR <= 16, "the cross-wave merge sums within one 16-lane DPP row");
    using VT = vf<VEC>;
    constexpr int RPW = 64 / LPR;
    constexpr int RPB = (WPR == 1) ? WAVES * RPW : WAVES / WPR;
    // Hold gamma/beta (or w) beside x only while x + parameters stay within a
    // quarter of the per-lane VGPR budget that WAVES-wide workgroups leave
    // (128 at 16 waves, 256 at 8, 512 below).
    constexpr int kParams = (OP == OP_LN) ? 2 : 1;
    constexpr int kBudget = WAVES >= 16 ? 128 : (WAVES >= 8 ? 256 : 512);
    constexpr bool PRELOAD = PRE >= 0 ? PRE == 1 : VEC * Q * (1 + kParams) <= kBudget / 4;
    constexpr bool PLDS = PRE == 2;
    constexpr bool MPAR = MRG >= 0 ? MRG == 1 : WPR >= 16;
    static_assert(!PLDS || (VEC >= 4 && !PEEL), "LDS parameters need the aligned 16-byte path");
    constexpr int kCapV = LPR * WPR * Q;  // 16-byte accesses per row the variant covers
    constexpr int kF4 = VEC >= 4 ? VEC / 4 : 1;  // float4 parameter words per access
    static_assert(!PLDS || kCapV * kF4 * kParams * 16 <= 64 * 1024, "LDS parameter stage too large");

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wr = (WPR == 1) ? 0 : wave % WPR;
    const int rib = (WPR == 1) ? wave * RPW + lane / LPR : wave / WPR;
    const int li = (WPR == 1) ? lane % LPR : lane;

    // (wave mean or sum of squares, wave M2) per row and wave: the one exchange
    __shared__ float2 xch[RPB][WPR];
    __shared__ f4 lds_par[PLDS ? kParams : 1][PLDS ? kCapV * kF4 : 1];

    const int d = p.d;
    const float eps = p.eps;
    const float inv_d = p.inv_d;

    if constexpr (PLDS) {
        // every lane of the workgroup copies part of gamma/beta into LDS; the
        // barrier before the output pass publishes it
        const int nv = d >> 2;
        for (int i = tid; i < nv && i < kCapV * kF4; i += WAVES * 64) {
            lds_par[0][i] = ld4<false>(p.p0 + 4 * i);
            if constexpr (OP == OP_LN) lds_par[kParams - 1][i] = ld4<false>(p.p1 + 4 * i);
        }
    }

    // one row group per workgroup: the grid covers every row once
    {
        // A row past the end (only in the last workgroup) re-reads the last
        // row and stores nothing, so every load below is in bounds without a
        // branch: loads are unconditional at clamped addresses, and values a
        // lane does not own are zeroed by selects.  Only stores are predicated.
        // every lane of the workgroup copies part of gamma/beta into LDS; a
    // barrier before the output pass publishes it.  16-bit rows stage them
    // ahead of the row's loads, float32 rows (one wave of sixteen slots)
    // behind them: each order measured 1-1.5% faster than the other there
    // (BF16 LayerNorm [4096,768] 4.00 against 4.06 us; float32 [4096,4096]
    // 22.10 against 22.33).
    auto stage_params = [&]() {
        const int nv = d >> 2;
        for (int i = tid; i < nv && i < kCapV * kF4; i += WAVES * 64) {
            lds_par[0][i] = ld4<false>(p.p0 + 4 * i);
            if constexpr (OP == OP_LN) lds_par[kParams - 1][i] = ld4<false>(p.p1 + 4 * i);
        }
    };
    if constexpr (PLDS && sizeof(T) == 2) stage_params();

    const int64_t row_raw = (int64_t)blockIdx.x * RPB + rib;
        const bool rv = row_raw < p.rows;
        const int64_t row = rv ? row_raw : p.rows - 1;
        const T *xr = static_cast<const T *>(p.x) + row * p.ldx;
        T *yr = static_cast<T *>(p.y) + row * p.ldy;
        const T *rr = RES ? static_cast<const T *>(p.r) + row * p.ldr : nullptr;
        T *hr = (RES && p.h) ? static_cast<T *>(p.h) + row * p.ldh : nullptr;

        // row geometry: h head scalars, nvec body accesses, t tail scalars.
        // A peeled row's body starts on a multiple of A elements (a 16-byte
        // access, or a 128-byte cache line, so that each wave-wide access
        // covers whole lines); h < A <= 64 head elements go to the lanes of
        // wave 0, and the body holds at most d / VEC accesses.
        int h = 0, t = 0, nvec;
        if constexpr (PEEL) {
            const int A = p.peel_align;
            const int mis = (int)((reinterpret_cast<uintptr_t>(xr) / sizeof(T)) & (A - 1));
            h = (A - mis) & (A - 1);
            nvec = (int)((unsigned)(d - h) / VEC);   // >= 1: d >= 128 > h + VEC
            t = d - h - VEC * nvec;
        } else {
            nvec = (int)((unsigned)d / VEC);  // >= 1 for these paths
        }

        // 1. issue every load of the row before using any.  Lane li of wave
        // rank wr holds access k = li + LPR*(wr + WPR*q) of the body; an
        // access past the body re-reads the body's last one.
        int kc[Q];
        bool ok[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int k = li + LPR * (wr + WPR * q);
            ok[q] = rv && k < nvec;
            kc[q] = k < nvec ? k : nvec - 1;
        }
        VT v[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            VT raw = ldv<T, VEC, NTL>(xr + h + VEC * kc[q]);
            if constexpr (RES) raw = as_stored<T>(raw + ldv<T, VEC, NTL>(rr + h + VEC * kc[q]));
            v[q] = ok[q] ? raw : VT(0.f);
        }
        float hx = 0.f, tx = 0.f;
        bool hok = false, tok = false;
        int hi = 0, ti = 0;
        float gh = 0.f, gt = 0.f, bh = 0.f, bt = 0.f;   // head/tail parameters
        if constexpr (PEEL) {
            hok = rv && wr == 0 && li < h;
            tok = rv && wr == 0 && li < t;
            hi = li < h ? li : 0;
            ti = h + VEC * nvec + li;
            ti = ti < d ? ti : d - 1;
            float rh = lde<T, false>(xr + hi), rt = lde<T, false>(xr + ti);
            if constexpr (RES) {
                rh = as_stored<T>(rh + lde<T, false>(rr + hi));
                rt = as_stored<T>(rt + lde<T, false>(rr + ti));
            }
            hx = hok ? rh : 0.f;
            tx = tok ? rt : 0.f;
            // fetched with the row: a load in the output pass would wait on
            // the stores issued before it (vmcnt counts both)
            gh = p.p0[hi];
            gt = p.p0[ti];
            if constexpr (OP == OP_LN) {
                bh = p.p1[hi];
                bt = p.p1[ti];
            }
        }
        if constexpr (RES) {
            // the sums leave as soon as they exist, overlapping the reductions;
            // every element is owned by one lane, so h may alias x or r
            if (hr) {
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    if (!ok[q]) continue;
                    stv<T, VEC, NTS>(hr + h + VEC * kc[q], v[q]);
                }
                if (hok) ste<T, false>(hr + hi, hx);
                if (tok) ste<T, false>(hr + ti, tx);
            }
        }

        // parameters for the output pass: fetched while x is in flight when
        // the register budget allows, else slot by slot in the output pass
        auto load_params = [&](int q, VT &gq, VT &bq) {
            if constexpr (PLDS && VEC == 4) {
                gq = lds_par[0][kc[q]];
                if constexpr (OP == OP_LN) bq = lds_par[kParams - 1][kc[q]];
            } else if constexpr (PLDS) {
                // an oct's eight parameters are two consecutive float4 words
                gq = __builtin_shufflevector(lds_par[0][2 * kc[q]], lds_par[0][2 * kc[q] + 1], 0, 1, 2, 3, 4, 5, 6, 7);
                if constexpr (OP == OP_LN)
                    bq = __builtin_shufflevector(lds_par[kParams - 1][2 * kc[q]], lds_par[kParams - 1][2 * kc[q] + 1],
                                                 0, 1, 2, 3, 4, 5, 6, 7);
            } else if constexpr (!PEEL) {
                gq = ldp<VEC>(p.p0 + VEC * kc[q]);
                if constexpr (OP == OP_LN) bq = ldp<VEC>(p.p1 + VEC * kc[q]);
            } else {
                // the body's phase in the row decides the parameters' phase
                gq = ldp_scalar<VEC>(p.p0 + h + VEC * kc[q]);
                if constexpr (OP == OP_LN) bq = ldp_scalar<VEC>(p.p1 + h + VEC * kc[q]);
            }
        };
        VT g[Q], b[Q];
        if constexpr (PRELOAD) {
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                b[q] = VT(0.f);
                load_params(q, g[q], b[q]);
            }
        }

        // elements held by wave rank w of this row (all lanes agree)
        auto wave_count = [&](int w) -> int {
            int n = 0;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int s = LPR * (w + WPR * q);
                const int c = nvec - s;
                n += c <= 0 ? 0 : (c >= LPR ? LPR : c);
            }
            n *= VEC;
            if (w == 0) n += h + t;
            return n;
        };

        float mu, rs;
        if constexpr (OP == OP_LN) {
            // 2. mean of what this wave holds
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < Q; ++q) s += hsum(v[q]);
            s += hx + tx;
            const float S = group_sum<LPR>(s);
            float mu_w;
            if constexpr (WPR == 1) {
                mu_w = S * inv_d;
            } else {
                const int n_w = wave_count(wr);
                mu_w = n_w > 0 ? S / (float)n_w : 0.f;
            }
            // 3. squared deviations around it, from the same registers
            float m = 0.f;
#pragma unroll
            for (int q = 0; q < Q; ++q) m += ok[q] ? csq(v[q], mu_w) : 0.f;
            m += hok ? csq(hx, mu_w) : 0.f;
            m += tok ? csq(tx, mu_w) : 0.f;
            const float M2_w = group_sum<LPR>(m);
            float M2;
            if constexpr (WPR == 1) {
                mu = mu_w;
                M2 = M2_w;
            } else {
                // one exchange: every wave's (mean, M2) meets in LDS behind one
                // barrier, then the Chan-Golub-LeVeque merge
                //   mu = sum_w n_w mu_w / d,  M2 = sum_w [M2_w + n_w (mu_w - mu)^2].
                // Every wave reads the same entries and adds them in the same
                // order, so all waves of the row hold the same mu and M2.
                if (li == 0) xch[rib][wr] = make_float2(mu_w, M2_w);
                __syncthreads();
                if constexpr (MPAR) {
                    // lane w < WPR takes wave w's entry; two 16-lane sums
                    const bool own = lane < WPR;
                    const float2 e = xch[rib][own ? lane : 0];
                    const float n_e = own ? (float)wave_count(lane) : 0.f;
                    mu = readlane(group_sum<16>(own ? n_e * e.x : 0.f), 0) * inv_d;
                    const float dm = e.x - mu;
                    M2 = readlane(group_sum<16>(own ? e.y + n_e * dm * dm : 0.f), 0);
                } else {
                    // every lane walks the WPR broadcast entries
                    float tot = 0.f;
#pragma unroll
                    for (int w = 0; w < WPR; ++w) tot += (float)wave_count(w) * xch[rib][w].x;
                    mu = tot * inv_d;
                    M2 = 0.f;
#pragma unroll
                    for (int w = 0; w < WPR; ++w) {
                        const float2 e = xch[rib][w];
                        const float dm = e.x - mu;
                        M2 += e.y + (float)wave_count(w) * dm * dm;
                    }
                }
            }
            rs = rsq(M2 * inv_d + eps);
        } else {
            float s2 = 0.f;
#pragma unroll
            for (int q = 0; q < Q; ++q) s2 += sq(v[q]);
            s2 += hx * hx + tx * tx;
            float S2 = group_sum<LPR>(s2);
            if constexpr (WPR > 1) {
                if (li == 0) xch[rib][wr] = make_float2(S2, 0.f);
                __syncthreads();
                if constexpr (MPAR) {
                    const bool own = lane < WPR;
                    const float e = xch[rib][own ? lane : 0].x;
                    S2 = readlane(group_sum<16>(own ? e : 0.f), 0);
                } else {
                    S2 = 0.f;
#pragma unroll
                    for (int w = 0; w < WPR; ++w) S2 += xch[rib][w].x;
                }
            }
            mu = 0.f;
            rs = rsq(S2 * inv_d + eps);
        }

        if constexpr (PLDS && WPR == 1) __syncthreads();  // the LDS parameters are complete
        if constexpr (PEEL && PRELOAD) {
            // every load has returned before the first store, so the output
            // pass holds no wait on a store still in flight: 7-9% on peeled
            // rows ([256,8193])
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                keep(g[q]);
                if constexpr (OP == OP_LN) keep(b[q]);
            }
            keep(gh);
            keep(gt);
            if constexpr (OP == OP_LN) {
                keep(bh);
                keep(bt);
            }
        }
        // 4. normalize, scale, shift; store from the same registers
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            VT gq, bq = VT(0.f);
            if constexpr (PRELOAD) {
                gq = g[q];
                bq = b[q];
            } else {
                load_params(q, gq, bq);
            }
            VT o;
            if constexpr (OP == OP_LN) o = (v[q] - mu) * rs * gq + bq;
            else o = v[q] * gq * rs;
            if (ok[q]) stv<T, VEC, NTS>(yr + h + VEC * kc[q], o);
        }
        if constexpr (PEEL) {
            const float oh = (OP == OP_LN) ? (hx - mu) * rs * gh + bh : hx * gh * rs;
            const float ot = (OP == OP_LN) ? (tx - mu) * rs * gt + bt : tx * gt * rs;
            if (hok) ste<T, false>(yr + hi, oh);
            if (tok) ste<T, false>(yr + ti, ot);
        }
        if (rv && wr == 0 && li == 0) {
            if (OP == OP_LN && p.mean) p.mean[row] = mu;
            if (p.rstd) p.rstd[row] = rs;
        }
    }
}

// ---------------------------------------------------------------------------
// Aligned held rows with buffer loads: the 16-byte vector path of norm_held
// (LPR = 64, no peel) with x (and r) and, unless staged in LDS, the
// parameters read through raw buffer instructions.  The row's resource
// spans exactly its d elements (none for a row past the end), and gfx950
// range-checks the whole offset (VGPR, SGPR and immediate): an access past
// the row reads zero.  So a lane keeps one VGPR offset, each slot's offset
// is a scalar, and the clamped addresses and zeroing selects of norm_held go
// away; one wave holding a 16 KiB float32 row drops from 147 to 99 VGPRs,
// which lets 16 such waves share a CU.  Stores are norm_held's predicated
// global stores.  Sums, merge and output expression are norm_held's, so for
// equal (WPR, Q) the outputs carry the same bits.

// a raw buffer over `bytes` bytes from `base` (stride 0; the fourth word is
// the 32-bit data format gfx950 expects of untyped buffer accesses)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_buffer(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// VEC elements of T (16 bytes) at byte offset voff + soff, widened to float32
template <typename T, int VEC, bool NT>
__device__ __forceinline__ vf<VEC> bldv(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u4 raw = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, NT ? 2 : 0));
    if constexpr (std::is_same_v<T, float>) {
        static_assert(VEC == 4, "four float32 per access");
        return __builtin_bit_cast(f4, raw);
    } else {
        static_assert(VEC == 8 && sizeof(T) == 2, "eight 16-bit elements per access");
        typedef T t8 __attribute__((ext_vector_type(8)));
        return __builtin_convertvector(__builtin_bit_cast(t8, raw), f8);
    }
}

// VEC float32 parameters at byte offset voff + soff
template <int VEC>
__device__ __forceinline__ vf<VEC> bldp(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const f4 a = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
    if constexpr (VEC == 4) {
        return a;
    } else {
        const f4 b = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff + 16, 0));
        return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

template <typename T, int OP, int VEC, int WPR, int Q, int WAVES, bool PLDS, bool RES>
__global__ __launch_bounds__(WAVES * 64)
void norm_aligned(NormParams p)
{
    static_assert(VEC == 4 || (VEC == 8 && sizeof(T) == 2), "16-byte accesses");
    static_assert(WAVES % WPR == 0 && WPR <= 16, "whole rows per workgroup");
    using VT = vf<VEC>;
    constexpr int RPB = WAVES / WPR;
    constexpr int kParams = (OP == OP_LN) ? 2 : 1;
    constexpr int kCapV = 64 * WPR * Q;
    constexpr int kF4 = VEC / 4;
    static_assert(!PLDS || kCapV * kF4 * kParams * 16 <= 64 * 1024, "LDS parameter stage too large");
    constexpr uint32_t kAcc = 16;           // bytes of one row access
    constexpr uint32_t kPar = VEC * 4;      // bytes of its parameters
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wr = (WPR == 1) ? 0 : wave % WPR;
    const int rib = (WPR == 1) ? wave : wave / WPR;
    __shared__ float2 xch[RPB][WPR];
    __shared__ f4 lds_par[PLDS ? kParams : 1][PLDS ? kCapV * kF4 : 1];

    const int d = p.d;
    const float eps = p.eps;
    const float inv_d = p.inv_d;
    const int nvec = (int)((unsigned)d / VEC);  // >= 1: d % VEC == 0, d >= VEC
    const uint32_t rbytes = (uint32_t)d * (uint32_t)sizeof(T);

    // every lane of the workgroup copies part of gamma/beta into LDS; a
    // barrier before the output pass publishes it.  16-bit rows stage them
    // ahead of the row's loads, float32 rows (one wave of sixteen slots)
    // behind them: each order measured 1-1.5% faster than the other there
    // (BF16 LayerNorm [4096,768] 4.00 against 4.06 us; float32 [4096,4096]
    // 22.10 against 22.33).
    auto stage_params = [&]() {
        const int nv = d >> 2;
        for (int i = tid; i < nv && i < kCapV * kF4; i += WAVES * 64) {
            lds_par[0][i] = ld4<false>(p.p0 + 4 * i);
            if constexpr (OP == OP_LN) lds_par[kParams - 1][i] = ld4<false>(p.p1 + 4 * i);
        }
    };
    if constexpr (PLDS && sizeof(T) == 2) stage_params();

    const int64_t row_raw = (int64_t)blockIdx.x * RPB + rib;
    const bool rv = row_raw < p.rows;
    const int64_t row = rv ? row_raw : 0;
    const uint32_t nb = rv ? rbytes : 0u;   // a row past the end reads zeros
    const uint32_t voff = (uint32_t)lane * kAcc;
    auto soff = [&](int q) -> uint32_t { return (uint32_t)(64 * (wr + WPR * q)) * kAcc; };
    int kc[Q];        // access index, clamped into the row for LDS and stores
    bool ok[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int k = lane + 64 * (wr + WPR * q);
        ok[q] = rv && k < nvec;
        kc[q] = k < nvec ? k : nvec - 1;
    }

    // 1. every load of the row before any use
    VT v[Q];
    {
        const auto rx = row_buffer(static_cast<const T *>(p.x) + row * p.ldx, nb);
#pragma unroll
        for (int q = 0; q < Q; ++q) v[q] = bldv<T, VEC, true>(rx, voff, soff(q));
    }
    VT w[RES ? Q : 1];
    if constexpr (RES) {
        const auto rr = row_buffer(static_cast<const T *>(p.r) + row * p.ldr, nb);
#pragma unroll
        for (int q = 0; q < Q; ++q) w[q] = bldv<T, VEC, true>(rr, voff, soff(q));
    }
    if constexpr (PLDS && sizeof(T) == 4) stage_params();
    if constexpr (RES) {
#pragma unroll
        for (int q = 0; q < Q; ++q) v[q] = as_stored<T>(v[q] + w[q]);
        // the sums leave as soon as they exist; every element is owned by one
        // lane, so h may alias x or r
        if (p.h) {
            T *hr = static_cast<T *>(p.h) + row * p.ldh;
#pragma unroll
            for (int q = 0; q < Q; ++q)
                if (ok[q]) stv<T, VEC, true>(hr + VEC * kc[q], v[q]);
        }
    }

    // elements held by wave rank w of the row (all lanes agree)
    auto wave_count = [&](int w) -> int {
        int n = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int c = nvec - 64 * (w + WPR * q);
            n += c <= 0 ? 0 : (c >= 64 ? 64 : c);
        }
        return n * VEC;
    };

    float mu, rs;
    if constexpr (OP == OP_LN) {
        // slots past the row read zero through the range check; masking
        // them anyway keeps the sums independent of that behaviour
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < Q; ++q) s += ok[q] ? hsum(v[q]) : 0.f;
        const float S = group_sum<64>(s);
        float mu_w;
        if constexpr (WPR == 1) {
            mu_w = S * inv_d;
        } else {
            const int n_w = wave_count(wr);
            mu_w = n_w > 0 ? S / (float)n_w : 0.f;
        }
        float m = 0.f;
#pragma unroll
        for (int q = 0; q < Q; ++q) m += ok[q] ? csq(v[q], mu_w) : 0.f;
        const float M2_w = group_sum<64>(m);
        float M2;
        if constexpr (WPR == 1) {
            mu = mu_w;
            M2 = M2_w;
        } else {
            if (lane == 0) xch[rib][wr] = make_float2(mu_w, M2_w);
            __syncthreads();
            if constexpr (WPR >= 16) {
                const bool own = lane < WPR;
                const float2 e = xch[rib][own ? lane : 0];
                const float n_e = own ? (float)wave_count(lane) : 0.f;
                mu = readlane(group_sum<16>(own ? n_e * e.x : 0.f), 0) * inv_d;
                const float dm = e.x - mu;
                M2 = readlane(group_sum<16>(own ? e.y + n_e * dm * dm : 0.f), 0);
            } else {
                float tot = 0.f;
#pragma unroll
                for (int w = 0; w < WPR; ++w) tot += (float)wave_count(w) * xch[rib][w].x;
                mu = tot * inv_d;
                M2 = 0.f;
#pragma unroll
                for (int w = 0; w < WPR; ++w) {
                    const float2 e = xch[rib][w];
                    const float dm = e.x - mu;
                    M2 += e.y + (float)wave_count(w) * dm * dm;
                }
            }
        }
        rs = rsq(M2 * inv_d + eps);
    } else {
        float s2 = 0.f;
#pragma unroll
        for (int q = 0; q < Q; ++q) s2 += ok[q] ? sq(v[q]) : 0.f;
        float S2 = group_sum<64>(s2);
        if constexpr (WPR > 1) {
            if (lane == 0) xch[rib][wr] = make_float2(S2, 0.f);
            __syncthreads();
            if constexpr (WPR >= 16) {
                const bool own = lane < WPR;
                const float e = xch[rib][own ? lane : 0].x;
                S2 = readlane(group_sum<16>(own ? e : 0.f), 0);
            } else {
                S2 = 0.f;
#pragma unroll
                for (int w = 0; w < WPR; ++w) S2 += xch[rib][w].x;
            }
        }
        mu = 0.f;
        rs = rsq(S2 * inv_d + eps);
    }

    // 4. normalize, scale, shift; store from the same registers
    if constexpr (PLDS && WPR == 1) __syncthreads();  // the LDS parameters are complete
    const auto rp0 = row_buffer(p.p0, (uint32_t)d * 4u);
    const auto rp1 = row_buffer(OP == OP_LN ? p.p1 : p.p0, (uint32_t)d * 4u);
    T *yr = static_cast<T *>(p.y) + row * p.ldy;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        VT gq, bq = VT(0.f);
        if constexpr (PLDS && VEC == 4) {
            gq = lds_par[0][kc[q]];
            if constexpr (OP == OP_LN) bq = lds_par[kParams - 1][kc[q]];
        } else if constexpr (PLDS) {
            // an oct's eight parameters are two consecutive float4 words
            gq = __builtin_shufflevector(lds_par[0][2 * kc[q]], lds_par[0][2 * kc[q] + 1], 0, 1, 2, 3, 4, 5, 6, 7);
            if constexpr (OP == OP_LN)
                bq = __builtin_shufflevector(lds_par[kParams - 1][2 * kc[q]], lds_par[kParams - 1][2 * kc[q] + 1],
                                             0, 1, 2, 3, 4, 5, 6, 7);
        } else {
            const uint32_t ps = (uint32_t)(64 * (wr + WPR * q)) * kPar;
            gq = bldp<VEC>(rp0, (uint32_t)lane * kPar, ps);
            if constexpr (OP == OP_LN) bq = bldp<VEC>(rp1, (uint32_t)lane * kPar, ps);
        }
        VT o;
        if constexpr (OP == OP_LN) o = (v[q] - mu) * rs * gq + bq;
        else o = v[q] * gq * rs;
        if (ok[q]) stv<T, VEC, true>(yr + VEC * kc[q], o);
    }
    if (rv && wr == 0 && lane == 0) {
        if (OP == OP_LN && p.mean) p.mean[row] = mu;
        if (p.rstd) p.rstd[row] = rs;
    }
}

// ---------------------------------------------------------------------------
// Multi-row held kernel: the 16-byte vector path of norm_held (LPR = 64, no
// peel) with RV rows held at once by every group of WPR waves.  A lane holds
// the same Q accesses, hence the same columns, of each of its RV rows, so one
// fetch of gamma/beta (or w) serves RV rows.  In norm_held every row fetches
// its own parameters; at float32 that is twice the row's own bytes through
// the CU's vector memory path (four times for a 16-bit row), which costs more
// than the row's HBM traffic once a launch runs many rows.
//
// The parameters are fetched for every slot in one batch once the
// statistics are known: fetched slot by slot between the predicated stores,
// each fetch's latency would be paid in turn.  keep() ties the batch ahead of
// the stores.
//
// Arithmetic and its order are norm_held's (the same sums, the same
// per-wave merge, the same output expression), so for equal (WPR, Q) the
// two kernels produce the same bits.  Rows of the group are grp*RV .. +RV-1
// within the workgroup's RPB rows; a row past the end re-reads the last row
// and stores nothing.


template <typename T, int OP, int VEC, int WPR, int Q, int RV, int WAVES, bool RES>
__global__ __launch_bounds__(WAVES * 64)
void norm_multi(NormParams p)
{
    static_assert(VEC == 4 || (VEC == 8 && sizeof(T) == 2), "16-byte accesses");
    static_assert(WAVES % WPR == 0 && WPR <= 8, "whole row groups per workgroup, walk merge");
    static_assert(RV >= 2, "several rows per wave group");
    using VT = vf<VEC>;
    constexpr int GPB = WAVES / WPR;  // wave groups per workgroup
    constexpr int RPB = GPB * RV;     // rows per workgroup
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wr = (WPR == 1) ? 0 : wave % WPR;
    const int grp = (WPR == 1) ? wave : wave / WPR;
    __shared__ float2 xch[WPR > 1 ? RPB : 1][WPR];

    const int d = p.d;
    const int nvec = (int)((unsigned)d / VEC);  // >= 1: d % VEC == 0, d >= VEC
    const float eps = p.eps;
    const float inv_d = p.inv_d;

    int kc[Q];
    bool okc[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int k = lane + 64 * (wr + WPR * q);
        okc[q] = k < nvec;
        kc[q] = okc[q] ? k : nvec - 1;
    }
    int64_t row[RV];
    bool rv[RV];
#pragma unroll
    for (int j = 0; j < RV; ++j) {
        const int64_t r = (int64_t)blockIdx.x * RPB + grp * RV + j;
        rv[j] = r < p.rows;
        row[j] = rv[j] ? r : p.rows - 1;
    }

    // 1. every load of the group's RV rows before any use
    VT v[RV][Q];
#pragma unroll
    for (int j = 0; j < RV; ++j) {
        const T *xr = static_cast<const T *>(p.x) + row[j] * p.ldx;
        const T *rr = RES ? static_cast<const T *>(p.r) + row[j] * p.ldr : nullptr;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            VT raw = ldv<T, VEC, true>(xr + VEC * kc[q]);
            if constexpr (RES) raw = as_stored<T>(raw + ldv<T, VEC, true>(rr + VEC * kc[q]));
            v[j][q] = okc[q] ? raw : VT(0.f);
        }
    }
    if constexpr (RES) {
        if (p.h) {
#pragma unroll
            for (int j = 0; j < RV; ++j) {
                T *hr = static_cast<T *>(p.h) + row[j] * p.ldh;
#pragma unroll
                for (int q = 0; q < Q; ++q)
                    if (okc[q] && rv[j]) stv<T, VEC, true>(hr + VEC * kc[q], v[j][q]);
            }
        }
    }

    // elements held by wave rank w of a row (all lanes agree)
    auto wave_count = [&](int w) -> int {
        int n = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int c = nvec - 64 * (w + WPR * q);
            n += c <= 0 ? 0 : (c >= 64 ? 64 : c);
        }
        return n * VEC;
    };

    // 2.-3. the statistics of each row, one exchange for all RV rows
    float mu[RV], rs[RV];
    if constexpr (OP == OP_LN) {
        float muw[RV], m[RV];
#pragma unroll
        for (int j = 0; j < RV; ++j) {
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < Q; ++q) s += hsum(v[j][q]);
            const float S = group_sum<64>(s);
            if constexpr (WPR == 1) {
                muw[j] = S * inv_d;
            } else {
                const int n_w = wave_count(wr);
                muw[j] = n_w > 0 ? S / (float)n_w : 0.f;
            }
        }
#pragma unroll
        for (int j = 0; j < RV; ++j) {
            float t = 0.f;
#pragma unroll
            for (int q = 0; q < Q; ++q) t += okc[q] ? csq(v[j][q], muw[j]) : 0.f;
            m[j] = group_sum<64>(t);
        }
        if constexpr (WPR == 1) {
#pragma unroll
            for (int j = 0; j < RV; ++j) {
                mu[j] = muw[j];
                rs[j] = rsq(m[j] * inv_d + eps);
            }
        } else {
            if (lane == 0) {
#pragma unroll
                for (int j = 0; j < RV; ++j) xch[grp * RV + j][wr] = make_float2(muw[j], m[j]);
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < RV; ++j) {
                float tot = 0.f;
#pragma unroll
                for (int w = 0; w < WPR; ++w) tot += (float)wave_count(w) * xch[grp * RV + j][w].x;
                mu[j] = tot * inv_d;
                float M2 = 0.f;
#pragma unroll
                for (int w = 0; w < WPR; ++w) {
                    const float2 e = xch[grp * RV + j][w];
                    const float dm = e.x - mu[j];
                    M2 += e.y + (float)wave_count(w) * dm * dm;
                }
                rs[j] = rsq(M2 * inv_d + eps);
            }
        }
    } else {
        float S2[RV];
#pragma unroll
        for (int j = 0; j < RV; ++j) {
            float s2 = 0.f;
#pragma unroll
            for (int q = 0; q < Q; ++q) s2 += sq(v[j][q]);
            S2[j] = group_sum<64>(s2);
        }
        if constexpr (WPR > 1) {
            if (lane == 0) {
#pragma unroll
                for (int j = 0; j < RV; ++j) xch[grp * RV + j][wr] = make_float2(S2[j], 0.f);
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < RV; ++j) {
                float t = 0.f;
#pragma unroll
                for (int w = 0; w < WPR; ++w) t += xch[grp * RV + j][w].x;
                S2[j] = t;
            }
        }
#pragma unroll
        for (int j = 0; j < RV; ++j) {
            mu[j] = 0.f;
            rs[j] = rsq(S2[j] * inv_d + eps);
        }
    }

    // 4. the parameters of every slot in one batch, then normalize, scale,
    // shift and store each row from the same registers.  With one wave per
    // row no barrier stands between the loads of x and the batch, and the
    // compiler hoists the batch above the reductions for RMSNorm and for
    // one-slot LayerNorm.  For RMSNorm rows of two or three slots that cost
    // 12-21% ([8192,768] 10.4 against 8.5 us, [8192,512] 7.3 against 6.4),
    // so there an empty asm ties each address to the last row's rstd; for
    // four slots and for one-slot LayerNorm the tie cost 2-3%.
    constexpr bool kTie = WPR == 1 && OP == OP_RMS && (Q == 2 || Q == 3);
    VT g[Q], b[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        int pk = kc[q];
        if constexpr (kTie) asm("" : "+v"(pk) : "v"(rs[RV - 1]));
        g[q] = ldp<VEC>(p.p0 + VEC * pk);
        b[q] = (OP == OP_LN) ? ldp<VEC>(p.p1 + VEC * pk) : VT(0.f);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        keep(g[q]);
        if constexpr (OP == OP_LN) keep(b[q]);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
#pragma unroll
        for (int j = 0; j < RV; ++j) {
            T *yr = static_cast<T *>(p.y) + row[j] * p.ldy;
            VT o;
            if constexpr (OP == OP_LN) o = (v[j][q] - mu[j]) * rs[j] * g[q] + b[q];
            else o = v[j][q] * g[q] * rs[j];
            if (okc[q] && rv[j]) stv<T, VEC, true>(yr + VEC * kc[q], o);
        }
    }
    if (wr == 0 && lane == 0) {
#pragma unroll
        for (int j = 0; j < RV; ++j) {
            if (!rv[j]) continue;
            if (OP == OP_LN && p.mean) p.mean[row[j]] = mu[j];
            if (p.rstd) p.rstd[row[j]] = rs[j];
        }
    }
}

// ---------------------------------------------------------------------------
// Streamed-row kernel for rows wider than the held variants cover: one
// workgroup per row, the row read in chunks, twice: the statistics, then the
// output.  VEC as above
// (no peel).  U accesses per lane per chunk are kept in flight.

template <int WAVES>
__device__ __forceinline__ float block_sum(float v, float (*red)[WAVES], int &slot, int wave, int lane) {
    v = group_sum<64>(v);
    if (lane == 0) red[slot][wave] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) t += red[slot][w];
    slot ^= 1;
    return t;
}

template <typename T, int OP, int VEC, int WAVES, int U, bool RES = false>
__global__ __launch_bounds__(WAVES * 64)
void norm_looped(NormParams p)
{
    static_assert(VEC == 1 || VEC == 4 || (VEC == 8 && sizeof(T) == 2), "VEC");
    using VT = vf<VEC>;
    constexpr int NT = WAVES * 64;  // threads per workgroup
    __shared__ float red[2][WAVES];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int d = p.d;
    const int nvec = (int)((unsigned)d / VEC);
    int slot = 0;

    auto load = [&](const T *xr, int k) -> VT { return ldv<T, VEC, false>(xr + VEC * k); };
    auto param = [&](const float *pr, int k) -> VT { return ldp<VEC>(pr + VEC * k); };

    for (int64_t row = blockIdx.x; row < p.rows; row += gridDim.x) {
        const T *xr = static_cast<const T *>(p.x) + row * p.ldx;
        T *yr = static_cast<T *>(p.y) + row * p.ldy;
        const T *rr = RES ? static_cast<const T *>(p.r) + row * p.ldr : nullptr;
        T *hr = (RES && p.h) ? static_cast<T *>(p.h) + row * p.ldh : nullptr;
        float mu = 0.f, rs;
        // the value at access k: x, or x + r; once pass 1 has written h (each
        // thread re-reads only what it stored itself) later passes read it
        // back, which stays right when h aliases x or r
        auto value = [&](int k, bool after_pass1) -> VT {
            if constexpr (RES) {
                if (after_pass1 && hr) return load(hr, k);
                return as_stored<T>(load(xr, k) + load(rr, k));
            } else {
                return load(xr, k);
            }
        };

        // pass 1: RMSNorm the sum of squares; LayerNorm each lane's count,
        // mean and centered sum of squares, the chunk in registers centered
        // on its own mean and merged into the lane's running pair (Chan,
        // Golub and LeVeque), so x is read once for the statistics
        float s = 0.f, ln_n = 0.f, ln_m = 0.f;
        for (int k0 = 0; k0 < nvec; k0 += NT * U) {
            VT v[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = k0 + tid + NT * u;
                ok[u] = k < nvec;
                v[u] = ok[u] ? value(k, false) : VT(0.f);
            }
            if constexpr (RES) {
                if (hr) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int k = k0 + tid + NT * u;
                        if (k >= nvec) continue;
                        stv<T, VEC, false>(hr + VEC * k, v[u]);
                    }
                }
            }
            if constexpr (OP == OP_LN) {
                float c = 0.f, cs = 0.f;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    c += ok[u] ? (float)VEC : 0.f;
                    cs += hsum(v[u]);
                }
                if (c > 0.f) {
                    const float cm = cs / c;
                    float c2 = 0.f;
#pragma unroll
                    for (int u = 0; u < U; ++u) c2 += ok[u] ? csq(v[u], cm) : 0.f;
                    const float n1 = ln_n + c;
                    const float dm = cm - ln_m;
                    ln_m += dm * (c / n1);
                    s += c2 + dm * dm * (ln_n * c / n1);
                    ln_n = n1;
                }
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) s += sq(v[u]);
            }
        }

        if constexpr (OP == OP_LN) {
            // the lanes' pairs merged: mean = sum n_l m_l / d, M2 = sum of
            // M2_l + n_l (m_l - mean)^2
            mu = block_sum<WAVES>(ln_n * ln_m, red, slot, wave, lane) * p.inv_d;
            const float dl = ln_m - mu;
            const float M2 = block_sum<WAVES>(s + ln_n * dl * dl, red, slot, wave, lane);
            rs = rsq(M2 * p.inv_d + p.eps);
        } else {
            const float S = block_sum<WAVES>(s, red, slot, wave, lane);
            rs = rsq(S * p.inv_d + p.eps);
        }

        // final pass: normalize and store
        for (int k0 = 0; k0 < nvec; k0 += NT * U) {
            VT v[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = k0 + tid + NT * u;
                ok[u] = k < nvec;
                v[u] = ok[u] ? value(k, true) : VT(0.f);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (!ok[u]) continue;
                const int k = k0 + tid + NT * u;
                VT o;
                if constexpr (OP == OP_LN) o = (v[u] - mu) * rs * param(p.p0, k) + param(p.p1, k);
                else o = v[u] * param(p.p0, k) * rs;
                stv<T, VEC, false>(yr + VEC * k, o);
            }
        }
        if (tid == 0) {
            if (OP == OP_LN && p.mean) p.mean[row] = mu;
            if (p.rstd) p.rstd[row] = rs;
        }
    }
}

}  // namespace minorm
