// bwd_table.hpp — the compiled backward variants (see bwd_kernels.hpp), one
// table per storage type, instantiated in bwd_variants_{f32,f16,bf16}.hip.
//
// Held variants run 8 waves per workgroup: WPR waves per row and 8 / WPR
// rows per step.
// Vector variants hold VW elements per access (4 float32, 8 of a 16-bit
// type), single-element variants 1.  A float32 or a 16-bit lane
// holds at most 8 or 4 vector accesses of x and dy plus float64 column sums,
// which 256 VGPRs (8-wave workgroups) hold without spilling.
#pragma once

#include "bwd_kernels.hpp"
#include "variant_table.hpp"

#define MI_BWD_HELD(T, DT, OPC, OPN, VEC, WPR, Q)                                               \
    Variant{OPN "_" #VEC "_w" #WPR "_q" #Q "_b8",                                                \
            mi_norm_variant_info{OPC, DT, VEC, 0, 0, 64, WPR, Q, 8, 8 / WPR,                     \
                                 (int64_t)VEC * 64 * WPR * Q, VEC > 1 ? 1 : 0, 1},               \
            reinterpret_cast<const void *>(                                                     \
                &norm_bwd_held<T, (OPC == MI_NORM_OP_LAYERNORM_BWD ? OP_LN : OP_RMS), VEC, WPR, Q, 8>)}

// streamed rows: the column-chunk kernel, 4 waves; single elements (8 per
// lane per row) on any layout, 16-byte accesses (two float32 or one 16-bit
// per lane per row) on aligned rows
#define MI_BWD_STREAM_V(T, DT, OPC, OPN, VEC, U)                                               \
    Variant{OPN "_" #VEC "_stream_b4_u" #U,                                                     \
            mi_norm_variant_info{OPC, DT, VEC, 0, 1, 64, 4, U, 4, 1, kUnbounded, VEC > 1 ? 1 : 0, 1}, \
            reinterpret_cast<const void *>(                                                     \
                &norm_bwd_chunks<T, (OPC == MI_NORM_OP_LAYERNORM_BWD ? OP_LN : OP_RMS), VEC, 4, U>)}
#define MI_BWD_STREAM_X(T, DT, OPC, OPN, VW, U) MI_BWD_STREAM_V(T, DT, OPC, OPN, VW, U)
#define MI_BWD_STREAM(T, DT, OPC, OPN, VW)                                                     \
    MI_BWD_STREAM_V(T, DT, OPC, OPN, 1, 8), MI_BWD_STREAM_X(T, DT, OPC, OPN, VW, MI_BWD_STREAM_U##VW)
#define MI_BWD_STREAM_U4 2
#define MI_BWD_STREAM_U8 1

// vector accesses: one wave per row with 1-4 slots, then 2, 4, 8 waves per
// row with 2-4 slots (float32 also 6 and 8 at 8 waves per row).  LayerNorm
// keeps two float64 sums per value, so its lanes hold at most 24 values
// (float32 up to 6 slots, 16-bit up to 3): more spilled past 256 VGPRs.
#define MI_BWD_Q123(T, DT, OPC, OPN, VW, WPR)                                                  \
    MI_BWD_HELD(T, DT, OPC, OPN, VW, WPR, 2), MI_BWD_HELD(T, DT, OPC, OPN, VW, WPR, 3)
#define MI_BWD_VEC_COMMON(T, DT, OPC, OPN, VW)                                                 \
    MI_BWD_HELD(T, DT, OPC, OPN, VW, 1, 1), MI_BWD_HELD(T, DT, OPC, OPN, VW, 1, 2),              \
    MI_BWD_HELD(T, DT, OPC, OPN, VW, 1, 3), MI_BWD_Q123(T, DT, OPC, OPN, VW, 2),                 \
    MI_BWD_Q123(T, DT, OPC, OPN, VW, 4), MI_BWD_Q123(T, DT, OPC, OPN, VW, 8)
#define MI_BWD_Q4(T, DT, OPC, OPN, VW)                                                         \
    MI_BWD_HELD(T, DT, OPC, OPN, VW, 1, 4), MI_BWD_HELD(T, DT, OPC, OPN, VW, 2, 4),              \
    MI_BWD_HELD(T, DT, OPC, OPN, VW, 4, 4), MI_BWD_HELD(T, DT, OPC, OPN, VW, 8, 4)
// float32: LayerNorm to 6 slots, RMSNorm to 8; 16-bit: LayerNorm to 3, RMSNorm to 4
#define MI_BWD_VEC_LN_4(T, DT, OPC, OPN)                                                       \
    MI_BWD_VEC_COMMON(T, DT, OPC, OPN, 4), MI_BWD_Q4(T, DT, OPC, OPN, 4),                        \
    MI_BWD_HELD(T, DT, OPC, OPN, 4, 8, 6)
#define MI_BWD_VEC_RMS_4(T, DT, OPC, OPN)                                                      \
    MI_BWD_VEC_LN_4(T, DT, OPC, OPN), MI_BWD_HELD(T, DT, OPC, OPN, 4, 8, 8)
#define MI_BWD_VEC_LN_8(T, DT, OPC, OPN) MI_BWD_VEC_COMMON(T, DT, OPC, OPN, 8)
#define MI_BWD_VEC_RMS_8(T, DT, OPC, OPN) MI_BWD_VEC_COMMON(T, DT, OPC, OPN, 8), MI_BWD_Q4(T, DT, OPC, OPN, 8)

// single-element accesses: any layout
#define MI_BWD_SCALAR(T, DT, OPC, OPN)                                                         \
    MI_BWD_HELD(T, DT, OPC, OPN, 1, 1, 1), MI_BWD_HELD(T, DT, OPC, OPN, 1, 1, 2),                \
    MI_BWD_HELD(T, DT, OPC, OPN, 1, 1, 4), MI_BWD_HELD(T, DT, OPC, OPN, 1, 1, 8),                \
    MI_BWD_HELD(T, DT, OPC, OPN, 1, 2, 4), MI_BWD_HELD(T, DT, OPC, OPN, 1, 2, 8),                \
    MI_BWD_HELD(T, DT, OPC, OPN, 1, 2, 16), MI_BWD_HELD(T, DT, OPC, OPN, 1, 4, 4),               \
    MI_BWD_HELD(T, DT, OPC, OPN, 1, 4, 8), MI_BWD_HELD(T, DT, OPC, OPN, 1, 4, 16),               \
    MI_BWD_HELD(T, DT, OPC, OPN, 1, 8, 4), MI_BWD_HELD(T, DT, OPC, OPN, 1, 8, 8),                \
    MI_BWD_HELD(T, DT, OPC, OPN, 1, 8, 16)

#define MI_BWD_DTYPE_TABLE(T, DT, VW, SFX)                                                     \
    MI_BWD_VEC_LN_##VW(T, DT, MI_NORM_OP_LAYERNORM_BWD, "lnbwd" SFX),                          \
    MI_BWD_SCALAR(T, DT, MI_NORM_OP_LAYERNORM_BWD, "lnbwd" SFX),                               \
    MI_BWD_STREAM(T, DT, MI_NORM_OP_LAYERNORM_BWD, "lnbwd" SFX, VW),                               \
    MI_BWD_VEC_RMS_##VW(T, DT, MI_NORM_OP_RMSNORM_BWD, "rmsbwd" SFX),                          \
    MI_BWD_SCALAR(T, DT, MI_NORM_OP_RMSNORM_BWD, "rmsbwd" SFX),                                \
    MI_BWD_STREAM(T, DT, MI_NORM_OP_RMSNORM_BWD, "rmsbwd" SFX, VW)
