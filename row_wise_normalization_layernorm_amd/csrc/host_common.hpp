// host_common.hpp — host-side helpers shared by the forward (mi_norm.hip) and
// backward (mi_norm_bwd.hip) dispatchers: the variant tables as one id
// space, alignment and element-size rules, and byte-extent overlap tests.
#pragma once

#include <cstdint>

#include "mi_norm_tuning.h"
#include "variant_table.hpp"

namespace minorm {

// defined in variants_*.hip and bwd_variants_*.hip
extern const VariantTable kTableF32, kTableF16, kTableBF16;           // forward
extern const VariantTable kBwdTableF32, kBwdTableF16, kBwdTableBF16;  // backward

namespace host {

// The tables in id order: forward float32, binary16, bfloat16, then the
// backward tables in the same type order.  Forward float32 ids come first so
// they do not move when other tables grow.
constexpr int kDtypes = 3;
constexpr int kTables = 2 * kDtypes;

// The widest row a problem may have (2^31 - 2^16 elements).  The kernels
// that stream a row walk it with an int32 element index stepped by at most
// a few thousand past its last value; this margin below 2^31 keeps every
// index and step of it representable.
constexpr int64_t kMaxD = INT32_MAX - 65535;

inline const VariantTable &table_at(int t) {
    switch (t) {
    case 0: return kTableF32;
    case 1: return kTableF16;
    case 2: return kTableBF16;
    case 3: return kBwdTableF32;
    case 4: return kBwdTableF16;
    default: return kBwdTableBF16;
    }
}
inline int table_base_at(int t) {
    int base = 0;
    for (int i = 0; i < t; ++i) base += table_at(i).n;
    return base;
}
// the forward table of a storage type, and the first id in it
inline const VariantTable &table(int dtype) { return table_at(dtype); }
inline int table_base(int dtype) { return table_base_at(dtype); }
// the backward table of a storage type, and the first id in it
inline const VariantTable &bwd_table(int dtype) { return table_at(kDtypes + dtype); }
inline int bwd_table_base(int dtype) { return table_base_at(kDtypes + dtype); }

inline int num_variants() { return table_base_at(kTables); }
inline const Variant *variant(int id) {
    if (id < 0) return nullptr;
    for (int t = 0; t < kTables; ++t) {
        if (id < table_at(t).n) return &table_at(t).v[id];
        id -= table_at(t).n;
    }
    return nullptr;
}

inline uintptr_t addr(const void *p) { return reinterpret_cast<uintptr_t>(p); }
inline bool aligned(const void *p, uintptr_t a) { return (addr(p) & (a - 1)) == 0; }
inline bool al16(const void *p) { return aligned(p, 16); }
inline bool al4(const void *p) { return aligned(p, 4); }
inline int64_t esize(int dtype) { return dtype == MI_NORM_F32 ? 4 : 2; }
// elements per vector access of the vector paths: 16 bytes of any storage type
inline int64_t vwidth(int dtype) { return 16 / esize(dtype); }

// byte ranges [lo, hi)
struct Ext {
    uintptr_t lo, hi;
};
inline bool meet(Ext a, Ext b) { return a.lo < b.hi && b.lo < a.hi; }
inline Ext vec_ext(const void *p, int64_t n, int64_t es) { return Ext{addr(p), addr(p) + (uintptr_t)(n * es)}; }
inline Ext rows_ext(const void *p, int64_t ld, int64_t rows, int64_t d, int64_t es) {
    return Ext{addr(p), addr(p) + (uintptr_t)(((rows - 1) * ld + d) * es)};
}

// Whether two row tensors of one problem share an element.  With equal
// strides and an element-multiple offset it is exact: b's rows then sit at
// column offset m = offset mod ld of a's row slots, and the two are disjoint
// exactly when [m, m + d) stays inside [d, ld).  Otherwise any overlap of
// their extents counts.
inline bool rows_meet(const void *a, int64_t lda, const void *b, int64_t ldb, int64_t rows, int64_t d,
                      int64_t es) {
    if (!meet(rows_ext(a, lda, rows, d, es), rows_ext(b, ldb, rows, d, es))) return false;
    if (lda != ldb) return true;
    const int64_t delta = (int64_t)(addr(b) - addr(a));
    if (delta % es != 0) return true;
    const int64_t m = ((delta / es) % lda + lda) % lda;
    return !(m >= d && m + d <= lda);
}

// smallest listed slot count q with cap_per_slot * q >= n, or 0
inline int pick_q(int64_t n, int64_t cap_per_slot, const int *qs, int nq) {
    for (int i = 0; i < nq; ++i)
        if (cap_per_slot * qs[i] >= n) return qs[i];
    return 0;
}

}  // namespace host
}  // namespace minorm
