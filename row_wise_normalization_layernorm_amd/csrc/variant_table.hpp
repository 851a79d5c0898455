// variant_table.hpp — the compiled kernel variants of libmi_norm.so.
//
// Each storage type's variants are instantiated in a translation unit of
// their own (variants_f32.hip, variants_f16.hip, variants_bf16.hip), so the
// three compile in parallel; mi_norm.hip walks the three tables as one.
#pragma once

#include <climits>
#include <cstdint>

#include "mi_norm_tuning.h"
#include "norm_kernels.hpp"

namespace minorm {

struct Variant {
    const char *name;
    mi_norm_variant_info info;
    const void *fn;
};

struct VariantTable {
    const Variant *v;
    int n;
};


constexpr int64_t kUnbounded = INT64_MAX;

// ABI op codes: bit 0 picks the normalization, op >= 2 fuses the residual add
constexpr int kOps = 4;
constexpr int kop(int op) { return op & 1; }       // OP_LN or OP_RMS
constexpr bool kres(int op) { return op >= 2; }

}  // namespace minorm

// Where a held variant's output pass gets its parameters (norm_held's PRE).
// Rows of a 16-bit type on the aligned vector path stage them in LDS once
// per workgroup when the workgroup holds at least two rows and the stage
// fits 64 KiB: per row, an oct's parameters are four times its own bytes,
// and fetching them per row cost 2-9% against staging them (MI355X;
// float32 rows at up to eight slots, at twice their bytes, gained nothing).
// The float32 one-wave rows of sixteen slots stage them too: there the
// output pass's parameter fetch was the last global round trip of a wave
// that holds a 16 KiB row.  Peeled rows fetch them with the row's loads
// where the register budget allows (norm_held's default), so that every
// load has returned before the first store: 7-9% on [256,8193].  Everything
// else reads them in the output pass.
constexpr int held_pre(int es, int vec, int peel, int lpr, int wpr, int q, int waves) {
    if (es == 2 && vec == 8 && !peel && lpr == 64 && waves / wpr >= 2 && wpr * q <= 16) return 2;
    if (es == 4 && vec == 4 && !peel && lpr == 64 && wpr == 1 && q == 16 && waves >= 2) return 2;
    if (peel) return -1;
    return 0;
}

// The kernel of a held variant.  Aligned vector rows of full waves run
// norm_aligned (buffer loads, same bits as norm_held); peeled, scalar and
// narrow rows run norm_held.  Every held variant streams x (and r) in and y
// (and h) out with non-temporal hints; the cross-wave merge follows
// norm_held's default.
template <typename T, int OP, int VEC, int PEEL, int LPR, int WPR, int Q, int WAVES, bool RES>
inline const void *held_kernel() {
    constexpr int PRE = held_pre((int)sizeof(T), VEC, PEEL, LPR, WPR, Q, WAVES);
    if constexpr (VEC > 1 && !PEEL && LPR == 64)
        return reinterpret_cast<const void *>(&minorm::norm_aligned<T, OP, VEC, WPR, Q, WAVES, PRE == 2, RES>);
    else
        return reinterpret_cast<const void *>(
            &minorm::norm_held<T, OP, VEC, (PEEL != 0), LPR, WPR, Q, WAVES, true, true, PRE, -1, RES>);
}

// T is the storage type, DT its mi_norm_dtype, OPN the name prefix.
#define MI_HELD(T, DT, OPC, OPN, VEC, PEEL, LPR, WPR, Q, WAVES)                                \
    Variant{OPN "_" #VEC "_p" #PEEL "_l" #LPR "_w" #WPR "_q" #Q "_b" #WAVES,                  \
            mi_norm_variant_info{OPC, DT, VEC, PEEL, 0, LPR, WPR, Q, WAVES,                     \
                                 (WPR == 1) ? WAVES * (64 / LPR) : WAVES / WPR,                 \
                                 (int64_t)VEC * LPR * WPR * Q + (PEEL ? VEC - 1 : 0),           \
                                 (VEC > 1 && !PEEL) ? 1 : 0, 1},                                \
            held_kernel<T, kop(OPC), VEC, PEEL, LPR, WPR, Q, WAVES, kres(OPC)>()}

// the same shape with 4 (or 8) and with 16 waves per workgroup
#define MI_HELD2(T, DT, OPC, OPN, VEC, PEEL, LPR, WPR, Q, WSMALL)                              \
    MI_HELD(T, DT, OPC, OPN, VEC, PEEL, LPR, WPR, Q, WSMALL),                                   \
    MI_HELD(T, DT, OPC, OPN, VEC, PEEL, LPR, WPR, Q, 16)

#define MI_LOOP(T, DT, OPC, OPN, VEC, WAVES, U)                                                \
    Variant{OPN "_" #VEC "_loop_b" #WAVES "_u" #U,                                              \
            mi_norm_variant_info{OPC, DT, VEC, 0, 1, 64, WAVES, U, WAVES, 1, kUnbounded,        \
                                 VEC > 1 ? 1 : 0, 1},                                           \
            reinterpret_cast<const void *>(&norm_looped<T, kop(OPC), VEC, WAVES, U, kres(OPC)>)}

// Multi-row variants (norm_multi): two rows per wave group sharing one fetch
// of the parameters, 4-wave workgroups (8 at 8 waves per row), on the aligned
// vector path.  Rows of a 16-bit type hold at most four slots: two rows of
// eight octs plus their parameters do not fit the registers of a 4-wave
// workgroup without spilling.
#define MI_MULTI(T, DT, OPC, OPN, VEC, WPR, Q, WAVES)                                           \
    Variant{OPN "_" #VEC "_r2_w" #WPR "_q" #Q "_b" #WAVES,                                      \
            mi_norm_variant_info{OPC, DT, VEC, 0, 0, 64, WPR, Q, WAVES, (WAVES / WPR) * 2,      \
                                 (int64_t)VEC * 64 * WPR * Q, 1, 2},                            \
            reinterpret_cast<const void *>(&norm_multi<T, kop(OPC), VEC, WPR, Q, 2, WAVES, kres(OPC)>)}
#define MI_MULTI_Q16(T, DT, OPC, OPN, VEC, WPR, WAVES)                                          \
    MI_MULTI(T, DT, OPC, OPN, VEC, WPR, 1, WAVES), MI_MULTI(T, DT, OPC, OPN, VEC, WPR, 2, WAVES), \
    MI_MULTI(T, DT, OPC, OPN, VEC, WPR, 3, WAVES), MI_MULTI(T, DT, OPC, OPN, VEC, WPR, 4, WAVES)
#define MI_MULTI_Q_4(T, DT, OPC, OPN, WPR, WAVES)                                                \
    MI_MULTI_Q16(T, DT, OPC, OPN, 4, WPR, WAVES), MI_MULTI(T, DT, OPC, OPN, 4, WPR, 6, WAVES),   \
    MI_MULTI(T, DT, OPC, OPN, 4, WPR, 8, WAVES)
#define MI_MULTI_Q_8(T, DT, OPC, OPN, WPR, WAVES) MI_MULTI_Q16(T, DT, OPC, OPN, 8, WPR, WAVES)
#define MI_MULTI_ALL(T, DT, VW, OPC, OPN)                                                          \
    MI_MULTI_Q_##VW(T, DT, OPC, OPN, 1, 4), MI_MULTI_Q_##VW(T, DT, OPC, OPN, 2, 4),                   \
    MI_MULTI_Q_##VW(T, DT, OPC, OPN, 4, 4), MI_MULTI_Q_##VW(T, DT, OPC, OPN, 8, 8)

// every (waves per row, slots) pair of a vector path (VW elements per access:
// 4 for float32, 8 for the 16-bit types, 16 bytes either way): slots 1, 2,
// 3, 4, 6, 8 for 1, 2, 4, 8 and 16 waves per row
#define MI_SLOTS(T, DT, VW, OPC, OPN, PEEL, WPR, WSMALL)                                           \
    MI_HELD2(T, DT, OPC, OPN, VW, PEEL, 64, WPR, 1, WSMALL),                                     \
    MI_HELD2(T, DT, OPC, OPN, VW, PEEL, 64, WPR, 2, WSMALL),                                     \
    MI_HELD2(T, DT, OPC, OPN, VW, PEEL, 64, WPR, 3, WSMALL),                                     \
    MI_HELD2(T, DT, OPC, OPN, VW, PEEL, 64, WPR, 4, WSMALL),                                     \
    MI_HELD2(T, DT, OPC, OPN, VW, PEEL, 64, WPR, 6, WSMALL),                                     \
    MI_SLOT8_##VW##_##PEEL(T, DT, OPC, OPN, WPR, WSMALL)
#define MI_SLOTS16(T, DT, VW, OPC, OPN, PEEL)                                                      \
    MI_HELD(T, DT, OPC, OPN, VW, PEEL, 64, 16, 1, 16), MI_HELD(T, DT, OPC, OPN, VW, PEEL, 64, 16, 2, 16), \
    MI_HELD(T, DT, OPC, OPN, VW, PEEL, 64, 16, 3, 16), MI_HELD(T, DT, OPC, OPN, VW, PEEL, 64, 16, 4, 16), \
    MI_HELD(T, DT, OPC, OPN, VW, PEEL, 64, 16, 6, 16) MI_SLOT16_8_##VW##_##PEEL(T, DT, OPC, OPN)

// Eight slots: 16-bit octs on the peeled path hold 8 x 8 values plus the
// peel's scalars, which does not fit the 128 VGPRs of a 16-wave workgroup
// (the fused variants spilled), so that path stops at six slots in 16-wave
// workgroups and the dispatcher caps it there.
#define MI_SLOT8_4_0(T, DT, OPC, OPN, WPR, WS) MI_HELD2(T, DT, OPC, OPN, 4, 0, 64, WPR, 8, WS)
#define MI_SLOT8_4_1(T, DT, OPC, OPN, WPR, WS) MI_HELD2(T, DT, OPC, OPN, 4, 1, 64, WPR, 8, WS)
#define MI_SLOT8_8_0(T, DT, OPC, OPN, WPR, WS) MI_HELD2(T, DT, OPC, OPN, 8, 0, 64, WPR, 8, WS)
#define MI_SLOT8_8_1(T, DT, OPC, OPN, WPR, WS) MI_HELD(T, DT, OPC, OPN, 8, 1, 64, WPR, 8, WS)
#define MI_SLOT16_8_4_0(T, DT, OPC, OPN) , MI_HELD(T, DT, OPC, OPN, 4, 0, 64, 16, 8, 16)
#define MI_SLOT16_8_4_1(T, DT, OPC, OPN) , MI_HELD(T, DT, OPC, OPN, 4, 1, 64, 16, 8, 16)
#define MI_SLOT16_8_8_0(T, DT, OPC, OPN) , MI_HELD(T, DT, OPC, OPN, 8, 0, 64, 16, 8, 16)
#define MI_SLOT16_8_8_1(T, DT, OPC, OPN)
#define MI_PATHV(T, DT, VW, OPC, OPN, PEEL)                                                        \
    MI_SLOTS(T, DT, VW, OPC, OPN, PEEL, 1, 4), MI_SLOTS(T, DT, VW, OPC, OPN, PEEL, 2, 4),               \
    MI_SLOTS(T, DT, VW, OPC, OPN, PEEL, 4, 4), MI_SLOTS(T, DT, VW, OPC, OPN, PEEL, 8, 8),               \
    MI_SLOTS16(T, DT, VW, OPC, OPN, PEEL)

// One wave per float32 LayerNorm row of up to 4096 elements holding sixteen
// 16-byte slots (norm_aligned: 99 VGPRs, 5 waves per SIMD), in 4-, 8- and
// 16-wave workgroups: the dispatcher's choice for rows of 3-4 K elements
// with 3072-4096 rows.  Other operations and storage types have none
// (16-bit octs would need twice the registers).
#define MI_WIDE16_4_MI_NORM_OP_LAYERNORM(T, DT, OPC, OPN)                                          \
    MI_HELD(T, DT, OPC, OPN, 4, 0, 64, 1, 16, 4), MI_HELD(T, DT, OPC, OPN, 4, 0, 64, 1, 16, 8),      \
    MI_HELD(T, DT, OPC, OPN, 4, 0, 64, 1, 16, 16),
#define MI_WIDE16_4_MI_NORM_OP_RMSNORM(T, DT, OPC, OPN)
#define MI_WIDE16_4_MI_NORM_OP_ADD_LAYERNORM(T, DT, OPC, OPN)
#define MI_WIDE16_4_MI_NORM_OP_ADD_RMSNORM(T, DT, OPC, OPN)
#define MI_WIDE16_8_MI_NORM_OP_LAYERNORM(T, DT, OPC, OPN)
#define MI_WIDE16_8_MI_NORM_OP_RMSNORM(T, DT, OPC, OPN)
#define MI_WIDE16_8_MI_NORM_OP_ADD_LAYERNORM(T, DT, OPC, OPN)
#define MI_WIDE16_8_MI_NORM_OP_ADD_RMSNORM(T, DT, OPC, OPN)

#define MI_OP_TABLE(T, DT, VW, OPC, OPN)                                                           \
    /* vectors, aligned, d % VW == 0; 16 or 32 lanes per row for narrow rows */                 \
    MI_HELD2(T, DT, OPC, OPN, VW, 0, 16, 1, 1, 4), MI_HELD2(T, DT, OPC, OPN, VW, 0, 32, 1, 1, 4), \
    MI_PATHV(T, DT, VW, OPC, OPN, 0),                                                               \
    MI_WIDE16_##VW##_##OPC(T, DT, OPC, OPN)                                                         \
    /* vector body with a per-row scalar head and tail: any d, rows in one phase */            \
    MI_PATHV(T, DT, VW, OPC, OPN, 1),                                                               \
    /* single-element accesses: any d, any element alignment */                                \
    MI_HELD2(T, DT, OPC, OPN, 1, 0, 16, 1, 1, 4), MI_HELD2(T, DT, OPC, OPN, 1, 0, 32, 1, 1, 4), \
    MI_HELD2(T, DT, OPC, OPN, 1, 0, 64, 1, 1, 4), MI_HELD2(T, DT, OPC, OPN, 1, 0, 64, 1, 2, 4), \
    MI_HELD2(T, DT, OPC, OPN, 1, 0, 64, 1, 4, 4), MI_HELD2(T, DT, OPC, OPN, 1, 0, 64, 1, 8, 4), \
    MI_HELD2(T, DT, OPC, OPN, 1, 0, 64, 4, 4, 4), MI_HELD2(T, DT, OPC, OPN, 1, 0, 64, 4, 8, 4), \
    MI_HELD2(T, DT, OPC, OPN, 1, 0, 64, 8, 8, 8),                                               \
    MI_HELD(T, DT, OPC, OPN, 1, 0, 64, 16, 8, 16), MI_HELD(T, DT, OPC, OPN, 1, 0, 64, 16, 16, 16), \
    /* streamed rows, any width */                                                             \
    MI_LOOP(T, DT, OPC, OPN, VW, 4, 4), MI_LOOP(T, DT, OPC, OPN, 1, 4, 8),                      \
    /* two rows per wave group, one fetch of the parameters for both */                       \
    MI_MULTI_ALL(T, DT, VW, OPC, OPN)

// ---------------------------------------------------------------------------
// The default table: the shapes the dispatcher can choose for some problem
// (checked over a dense grid of operations, storage types, layouts, widths
// and row counts), kept whole per (waves per row, slots) where the
// workgroup-size rule reaches one size of a pair for only some of them.
// Builds with MI_NORM_FULL_TABLE defined compile MI_OP_TABLE above instead,
// every (waves per row, slots, workgroup) pair, for sweeps that force
// variants the dispatcher does not choose.
//   vectors, aligned: one wave 1-4, 6, 8 slots; two waves 1-4, 6, 8; four and
//     eight waves 1-4 (one slot in the smaller workgroup only); 16 waves 1-8
//   peeled: one wave 1-4; two, four, eight waves as the aligned path; 16 waves
//   two rows per wave group: float32 one wave 1-4, two waves 3, 4, 6, 8;
//     four and eight waves 3, 4 (16-bit: two, four, eight waves 3, 4)
#define MI_D_H4(T, DT, OPC, OPN, VW, PEEL, WPR, WS)                                                 \
    MI_HELD(T, DT, OPC, OPN, VW, PEEL, 64, WPR, 1, WS), MI_HELD2(T, DT, OPC, OPN, VW, PEEL, 64, WPR, 2, WS), \
    MI_HELD2(T, DT, OPC, OPN, VW, PEEL, 64, WPR, 3, WS), MI_HELD2(T, DT, OPC, OPN, VW, PEEL, 64, WPR, 4, WS)
#define MI_D_W1(T, DT, OPC, OPN, VW, PEEL)                                                          \
    MI_HELD2(T, DT, OPC, OPN, VW, PEEL, 64, 1, 1, 4), MI_HELD2(T, DT, OPC, OPN, VW, PEEL, 64, 1, 2, 4), \
    MI_HELD2(T, DT, OPC, OPN, VW, PEEL, 64, 1, 3, 4), MI_HELD2(T, DT, OPC, OPN, VW, PEEL, 64, 1, 4, 4)
#define MI_D_Q68(T, DT, OPC, OPN, VW, WPR)                                                          \
    MI_HELD2(T, DT, OPC, OPN, VW, 0, 64, WPR, 6, 4), MI_HELD2(T, DT, OPC, OPN, VW, 0, 64, WPR, 8, 4)
#define MI_D_MULTI_4(T, DT, OPC, OPN)                                                               \
    MI_MULTI_Q16(T, DT, OPC, OPN, 4, 1, 4),                                                          \
    MI_MULTI(T, DT, OPC, OPN, 4, 2, 3, 4), MI_MULTI(T, DT, OPC, OPN, 4, 2, 4, 4),                   \
    MI_MULTI(T, DT, OPC, OPN, 4, 2, 6, 4), MI_MULTI(T, DT, OPC, OPN, 4, 2, 8, 4),                   \
    MI_MULTI(T, DT, OPC, OPN, 4, 4, 3, 4), MI_MULTI(T, DT, OPC, OPN, 4, 4, 4, 4),                   \
    MI_MULTI(T, DT, OPC, OPN, 4, 8, 3, 8), MI_MULTI(T, DT, OPC, OPN, 4, 8, 4, 8)
#define MI_D_MULTI_8(T, DT, OPC, OPN)                                                               \
    MI_MULTI(T, DT, OPC, OPN, 8, 2, 3, 4), MI_MULTI(T, DT, OPC, OPN, 8, 2, 4, 4),                   \
    MI_MULTI(T, DT, OPC, OPN, 8, 4, 3, 4), MI_MULTI(T, DT, OPC, OPN, 8, 4, 4, 4),                   \
    MI_MULTI(T, DT, OPC, OPN, 8, 8, 3, 8), MI_MULTI(T, DT, OPC, OPN, 8, 8, 4, 8)

#define MI_D_OP_TABLE(T, DT, VW, OPC, OPN)                                                         \
    MI_HELD2(T, DT, OPC, OPN, VW, 0, 16, 1, 1, 4), MI_HELD2(T, DT, OPC, OPN, VW, 0, 32, 1, 1, 4), \
    MI_D_W1(T, DT, OPC, OPN, VW, 0), MI_D_Q68(T, DT, OPC, OPN, VW, 1),                              \
    MI_D_H4(T, DT, OPC, OPN, VW, 0, 2, 4), MI_D_Q68(T, DT, OPC, OPN, VW, 2),                        \
    MI_D_H4(T, DT, OPC, OPN, VW, 0, 4, 4), MI_D_H4(T, DT, OPC, OPN, VW, 0, 8, 8),                   \
    MI_SLOTS16(T, DT, VW, OPC, OPN, 0),                                                             \
    MI_WIDE16_##VW##_##OPC(T, DT, OPC, OPN)                                                         \
    MI_D_W1(T, DT, OPC, OPN, VW, 1),                                                                \
    MI_D_H4(T, DT, OPC, OPN, VW, 1, 2, 4), MI_D_H4(T, DT, OPC, OPN, VW, 1, 4, 4),                   \
    MI_D_H4(T, DT, OPC, OPN, VW, 1, 8, 8), MI_SLOTS16(T, DT, VW, OPC, OPN, 1),                      \
    MI_HELD2(T, DT, OPC, OPN, 1, 0, 16, 1, 1, 4), MI_HELD2(T, DT, OPC, OPN, 1, 0, 32, 1, 1, 4), \
    MI_HELD2(T, DT, OPC, OPN, 1, 0, 64, 1, 1, 4), MI_HELD2(T, DT, OPC, OPN, 1, 0, 64, 1, 2, 4), \
    MI_HELD2(T, DT, OPC, OPN, 1, 0, 64, 1, 4, 4), MI_HELD2(T, DT, OPC, OPN, 1, 0, 64, 1, 8, 4), \
    MI_HELD2(T, DT, OPC, OPN, 1, 0, 64, 4, 4, 4), MI_HELD2(T, DT, OPC, OPN, 1, 0, 64, 4, 8, 4), \
    MI_HELD2(T, DT, OPC, OPN, 1, 0, 64, 8, 8, 8),                                               \
    MI_HELD(T, DT, OPC, OPN, 1, 0, 64, 16, 8, 16), MI_HELD(T, DT, OPC, OPN, 1, 0, 64, 16, 16, 16), \
    MI_LOOP(T, DT, OPC, OPN, VW, 4, 4), MI_LOOP(T, DT, OPC, OPN, 1, 4, 8),                      \
    MI_D_MULTI_##VW(T, DT, OPC, OPN)

#ifdef MI_NORM_FULL_TABLE
#define MI_TABLE_OF MI_OP_TABLE
#else
#define MI_TABLE_OF MI_D_OP_TABLE
#endif

// the four operations of one storage type; VW its vector width in
// elements, SFX its name suffix
#define MI_DTYPE_TABLE(T, DT, VW, SFX)                                                             \
    MI_TABLE_OF(T, DT, VW, MI_NORM_OP_LAYERNORM, "ln" SFX),                                         \
    MI_TABLE_OF(T, DT, VW, MI_NORM_OP_RMSNORM, "rms" SFX),                                          \
    MI_TABLE_OF(T, DT, VW, MI_NORM_OP_ADD_LAYERNORM, "addln" SFX),                                  \
    MI_TABLE_OF(T, DT, VW, MI_NORM_OP_ADD_RMSNORM, "addrms" SFX)
