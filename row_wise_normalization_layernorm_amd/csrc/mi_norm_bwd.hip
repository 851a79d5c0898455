// mi_norm_bwd.hip — libmi_norm.so: dispatch, validation and the C ABI of the
// LayerNorm / RMSNorm backward (include/mi_norm.h, "Backward"), over the
// tables of bwd_variants_{f32,f16,bf16}.hip.
//
// A call runs the row kernel (dx, and each workgroup's partial sums of the
// parameter gradients) and then the column reduction of the partial rows;
// rows wider than the held variants run the per-row statistics kernel first
// and a column-chunk kernel in place of the row kernel.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "bwd_kernels.hpp"
#include "host_common.hpp"
#include "mi_norm_tuning.h"

using namespace minorm;
using namespace minorm::host;

// The workspace of mi_norm_bwd_noalloc: one array per GPU, held from the
// moment the library's code is loaded on that GPU until the process ends.
// Host code never uses this name as an address: each device's address comes
// from hipGetSymbolAddress (scratch_ptr below).
constexpr int64_t kScratchBytes = int64_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// partial rows: workgroups of the row kernel (one per CU), row blocks of the
// streamed path.  Measured on MI355X: 512 took LayerNorm backward [4096,768]
// 15.4 us (13.5 with 256), BF16 15.5 (11.6); 128 left half the CUs idle
// ([32768,8192] 729 us against 560).
constexpr int64_t kMaxPartials = 256;
constexpr int64_t kAlign = 256;        // workspace alignment and section alignment
constexpr int64_t kMaxGrid = 1 << 20;  // grid cap of the statistics kernel's row loop
constexpr int kRowstatsU = 4;          // norm_bwd_rowstats: accesses per lane in flight

inline int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }
inline int64_t dpad_of(int64_t d) { return (d + 3) & ~int64_t(3); }
inline bool is_ln(const mi_norm_bwd_problem &P) { return P.op == MI_NORM_OP_LAYERNORM; }
inline int bwd_opcode(int op) { return op == MI_NORM_OP_LAYERNORM ? MI_NORM_OP_LAYERNORM_BWD : MI_NORM_OP_RMSNORM_BWD; }
inline bool want_pg(const mi_norm_bwd_problem &P) {
    return P.dparams0 != nullptr || (is_ln(P) && P.dparams1 != nullptr);
}
inline int ngrads(const mi_norm_bwd_problem &P) { return is_ln(P) ? 2 : 1; }

// dy, x, dx with their row strides (0 resolved to d; any stride of a one-row
// problem reads as d)
struct BRows {
    const void *p[3];
    int64_t ld[3];
};
BRows brows_of(const mi_norm_bwd_problem &P) {
    BRows R{{P.dy, P.x, P.dx}, {P.lddy, P.ldx, P.lddx}};
    for (int i = 0; i < 3; ++i)
        if (R.ld[i] == 0 || P.rows <= 1) R.ld[i] = P.d;
    return R;
}

// workspace sections: partial rows, then per-row statistics
int64_t part_bytes(const mi_norm_bwd_problem &P) {
    return want_pg(P) ? align_up(kMaxPartials * ngrads(P) * dpad_of(P.d) * 4, kAlign) : 0;
}
int64_t stats_bytes(const mi_norm_bwd_problem &P) { return align_up(P.rows * 8, kAlign); }

bool bshape_ok(const mi_norm_bwd_problem &P) {
    if ((P.op != MI_NORM_OP_LAYERNORM && P.op != MI_NORM_OP_RMSNORM) || P.dtype < 0 || P.dtype >= kDtypes)
        return false;
    if (!P.dy || !P.x || !P.dx || !P.params0 || !P.rstd || (is_ln(P) && !P.mean)) return false;
    if (P.d < 1 || P.d > kMaxD || P.rows < 0) return false;
    for (const void *q : {(const void *)P.params0, (const void *)P.rstd, (const void *)(is_ln(P) ? P.mean : nullptr),
                          (const void *)P.dparams0, (const void *)(is_ln(P) ? P.dparams1 : nullptr)})
        if (q && !al4(q)) return false;
    const int64_t es = esize(P.dtype);
    const int64_t raw[3] = {P.lddy, P.ldx, P.lddx};
    const BRows R = brows_of(P);
    for (int i = 0; i < 3; ++i) {
        if (!aligned(R.p[i], (uintptr_t)es) || raw[i] < 0) return false;
        if (P.rows > 1 && R.ld[i] < P.d) return false;
        if (P.rows > 1 && R.ld[i] > (INT64_MAX / es - P.d) / (P.rows - 1)) return false;
    }
    if (P.rows > INT64_MAX / 64) return false;
    return true;
}

int64_t workspace_needed(const mi_norm_bwd_problem &P) { return part_bytes(P) + stats_bytes(P); }

// the workspace bytes of *p, or -1 when its op, type or shape is invalid
int64_t workspace_needed_checked(const mi_norm_bwd_problem &P) {
    if ((P.op != MI_NORM_OP_LAYERNORM && P.op != MI_NORM_OP_RMSNORM) || P.dtype < 0 || P.dtype >= kDtypes ||
        P.d < 1 || P.d > kMaxD || P.rows < 0 || P.rows > INT64_MAX / 64)
        return -1;
    return workspace_needed(P);
}

// every row tensor 16-byte aligned, strides and d multiples of the vector
// width, gamma (w) 16-byte aligned: the vector path
bool vec_layout(const mi_norm_bwd_problem &P) {
    const int64_t W = vwidth(P.dtype);
    if (P.d % W != 0 || !al16(P.params0)) return false;
    const BRows R = brows_of(P);
    for (int i = 0; i < 3; ++i)
        if (!al16(R.p[i]) || R.ld[i] % W != 0) return false;
    return true;
}

int find_bwd(int op, int dt, int vec, int looped, int wpr, int q, int waves = 8) {
    const VariantTable &T = bwd_table(dt);
    for (int i = 0; i < T.n; ++i) {
        const mi_norm_variant_info &v = T.v[i].info;
        if (v.op != bwd_opcode(op) || v.vec != vec || v.looped != looped) continue;
        if (looped || (v.waves_per_row == wpr && v.slots == q && v.waves_per_block == waves))
            return bwd_table_base(dt) + i;
    }
    return -1;
}

// The most slots a vector variant of this op and type holds: LayerNorm's
// lanes keep two float64 sums per value and stop at 24 values (float32 6
// slots, 16-bit 3); RMSNorm's one sum allows 32 (8 and 4).
int max_slots(int op, int W) {
    if (op == MI_NORM_OP_LAYERNORM) return W == 4 ? 6 : 3;
    return W == 4 ? 8 : 4;
}

// One wave per row while up to four (at most max_slots) slots hold it.
// Wider rows take the fewest of 2 and 4 waves whose lanes hold them in at
// most three float32 slots or two 16-bit ones (12 or 16 values, which the
// pipelined loop of norm_bwd_held keeps two of), else 8 waves with up to
// max_slots; single-element rows likewise with 1-8 slots for one wave, 4-16
// for more.  Measured with the pipelined loop (8-wave workgroups): LayerNorm
// [4096,2048] 24.0 us at four waves of two slots against 24.1 at two of
// four, [65536,2048] 263 against 278, [8192,4096] 71.0 against 73.1; RMSNorm
// [8192,4096] 67.7 against 70.3; BF16 RMSNorm [8192,8192] 70.8 against 77.0,
// [16384,4096] 69.1 against 75.4, BF16 LayerNorm [4096,6144] 37.1 against
// 42.1.  16-wave workgroups, which had doubled the rows in flight per CU
// before the pipelined loop, now ran no faster (LayerNorm [4096,3072] 32.9
// against 36.6, [8192,4096] 71.0 against 72.5).
int select_bwd(const mi_norm_bwd_problem &P) {
    if (!bshape_ok(P)) return -1;
    const int op = P.op, dt = P.dtype;
    if (vec_layout(P)) {
        const int W = (int)vwidth(dt);
        const int64_t nvec = P.d / W;
        const int qmax = max_slots(op, W);
        const int q4 = qmax < 4 ? qmax : 4;
        static const int qs[] = {1, 2, 3, 4, 6, 8};
        const int nq = qmax == 3 ? 3 : (qmax == 4 ? 4 : (qmax == 6 ? 5 : 6));
        int wpr = 0, q = 0;
        if (nvec <= 64 * q4) {
            wpr = 1;
            q = pick_q(nvec, 64, qs, q4 == 3 ? 3 : 4);
        } else {
            const int c = W == 4 ? 3 : 2;   // slots of the pipelined rows of 2 and 4 waves
            wpr = nvec <= 128 * c ? 2 : (nvec <= 256 * c ? 4 : 8);
            q = pick_q(nvec, 64 * wpr, qs + 1, (wpr == 8 ? nq : c) - 1);
        }
        if (q) return find_bwd(op, dt, W, 0, wpr, q);
        return find_bwd(op, dt, W, 1, 0, 0);
    }
    const int64_t n = P.d;
    static const int s1[] = {1, 2, 4, 8};
    static const int sw[] = {4, 8, 16};
    if (n <= 512) return find_bwd(op, dt, 1, 0, 1, pick_q(n, 64, s1, 4));
    const int wpr = n <= 2048 ? 2 : (n <= 4096 ? 4 : 8);
    const int q = pick_q(n, 64 * wpr, sw, 3);
    if (q) return find_bwd(op, dt, 1, 0, wpr, q);
    return find_bwd(op, dt, 1, 1, 0, 0);
}

bool eligible_bwd(int id, const mi_norm_bwd_problem &P) {
    const Variant *V = variant(id);
    if (!V || !bshape_ok(P)) return false;
    const mi_norm_variant_info &v = V->info;
    if (v.op != bwd_opcode(P.op) || v.dtype != P.dtype) return false;
    if (v.looped) return v.vec == 1 || vec_layout(P);
    if (v.vec > 1) return vec_layout(P) && P.d <= v.max_d;
    return P.d <= v.max_d;
}

// dx is dy or x (same pointer and stride) or shares no element with them and
// meets no float32 input; the parameter gradients and the workspace meet
// nothing else
bool aliasing_bwd(const mi_norm_bwd_problem &P, int64_t ws_bytes) {
    const int64_t es = esize(P.dtype), rows = P.rows, d = P.d;
    const bool ln = is_ln(P);
    const BRows R = brows_of(P);
    Ext ins[3];
    int nins = 0;
    ins[nins++] = vec_ext(P.params0, d, 4);
    ins[nins++] = vec_ext(P.rstd, rows, 4);
    if (ln) ins[nins++] = vec_ext(P.mean, rows, 4);
    if (rows > 0) {
        for (int t = 0; t < 2; ++t) {
            if (R.p[t] == R.p[2] && R.ld[t] == R.ld[2]) continue;  // in place
            if (rows_meet(R.p[2], R.ld[2], R.p[t], R.ld[t], rows, d, es)) return false;
        }
        const Ext edx = rows_ext(R.p[2], R.ld[2], rows, d, es);
        for (int i = 0; i < nins; ++i)
            if (rows > 0 && meet(edx, ins[i])) return false;
    }
    // the outputs that are plain byte ranges
    Ext outs[3];
    int nouts = 0;
    if (P.dparams0) outs[nouts++] = vec_ext(P.dparams0, d, 4);
    if (ln && P.dparams1) outs[nouts++] = vec_ext(P.dparams1, d, 4);
    if (ws_bytes > 0) outs[nouts++] = vec_ext(P.workspace, ws_bytes, 1);
    for (int o = 0; o < nouts; ++o) {
        for (int j = o + 1; j < nouts; ++j)
            if (meet(outs[o], outs[j])) return false;
        for (int i = 0; i < nins; ++i)
            if (meet(outs[o], ins[i])) return false;
        if (rows > 0)
            for (int t = 0; t < 3; ++t)
                if (meet(outs[o], rows_ext(R.p[t], R.ld[t], rows, d, es))) return false;
    }
    return true;
}

mi_norm_status validate_bwd(const mi_norm_bwd_problem &P) {
    if (!bshape_ok(P)) return MI_NORM_ERR_INVALID;
    const int64_t need = workspace_needed(P);
    const int sel = select_bwd(P);
    const bool uses_ws = want_pg(P) || (sel >= 0 && variant(sel)->info.looped);
    if (uses_ws && (!P.workspace || P.workspace_bytes < need)) return MI_NORM_ERR_INVALID;
    if (P.workspace && !aligned(P.workspace, kAlign)) return MI_NORM_ERR_INVALID;
    if (!aliasing_bwd(P, P.workspace ? need : 0)) return MI_NORM_ERR_INVALID;
    return MI_NORM_OK;
}

// the per-row statistics kernel of the streamed path, with the chunk
// kernel's access width (vec 1, or 16 bytes)
template <typename T, int VEC>
const void *rowstats_of(bool ln) {
    return ln ? reinterpret_cast<const void *>(&norm_bwd_rowstats<T, OP_LN, VEC, 4, kRowstatsU>)
              : reinterpret_cast<const void *>(&norm_bwd_rowstats<T, OP_RMS, VEC, 4, kRowstatsU>);
}
const void *rowstats_fn(int dtype, bool ln, int vec) {
    switch (dtype) {
    case MI_NORM_F32: return vec > 1 ? rowstats_of<float, 4>(ln) : rowstats_of<float, 1>(ln);
    case MI_NORM_F16: return vec > 1 ? rowstats_of<_Float16, 8>(ln) : rowstats_of<_Float16, 1>(ln);
    default: return vec > 1 ? rowstats_of<__bf16, 8>(ln) : rowstats_of<__bf16, 1>(ln);
    }
}

mi_norm_status launch_reduce(const mi_norm_bwd_problem &P, const float *part, int64_t nblk, hipStream_t stream) {
    int32_t d = (int32_t)P.d, dpad = (int32_t)dpad_of(P.d);
    float *o0 = P.dparams0;
    float *o1 = is_ln(P) ? P.dparams1 : nullptr;
    void *args[] = {&part, &nblk, &d, &dpad, &o0, &o1};
    const dim3 grid((unsigned)((dpad + 15) / 16), (unsigned)ngrads(P));  // 16 columns per workgroup
    const void *fn = is_ln(P) ? reinterpret_cast<const void *>(&norm_bwd_reduce<2>)
                              : reinterpret_cast<const void *>(&norm_bwd_reduce<1>);
    return hipLaunchKernel(fn, grid, dim3(256), args, 0, stream) == hipSuccess ? MI_NORM_OK : MI_NORM_ERR_HIP;
}

mi_norm_status run_bwd(int forced, const mi_norm_bwd_problem &P, hipStream_t stream) {
    const mi_norm_status st = validate_bwd(P);
    if (st != MI_NORM_OK) return st;
    int id = forced;
    if (id < 0) {
        id = select_bwd(P);
        if (id < 0) return MI_NORM_ERR_INVALID;
    } else if (!eligible_bwd(id, P)) {
        return MI_NORM_ERR_INVALID;
    }
    const Variant &V = *variant(id);
    if (V.info.looped && !(P.workspace && aligned(P.workspace, kAlign) && P.workspace_bytes >= workspace_needed(P)))
        return MI_NORM_ERR_INVALID;  // a forced streamed variant needs the statistics section
    const bool pg = want_pg(P);
    if (P.rows == 0) {
        // no rows: dx is empty and the parameter gradients are zero sums
        return pg ? launch_reduce(P, nullptr, 0, stream) : MI_NORM_OK;
    }
    const BRows R = brows_of(P);
    BwdParams K;
    K.dy = R.p[0];
    K.x = R.p[1];
    K.dx = const_cast<void *>(R.p[2]);
    K.lddy = R.ld[0];
    K.ldx = R.ld[1];
    K.lddx = R.ld[2];
    K.p0 = P.params0;
    K.mean = is_ln(P) ? P.mean : nullptr;
    K.rstd = P.rstd;
    K.part = pg ? static_cast<float *>(P.workspace) : nullptr;
    K.stats = P.workspace ? reinterpret_cast<float2 *>(static_cast<char *>(P.workspace) + part_bytes(P)) : nullptr;
    K.rows = P.rows;
    K.d = (int32_t)P.d;
    K.dpad = (int32_t)dpad_of(P.d);
    K.inv_d = 1.0 / (double)P.d;
    int64_t nblk;
    if (!V.info.looped) {
        const int64_t rpb = V.info.rows_per_block;
        const int64_t groups = (P.rows + rpb - 1) / rpb;
        nblk = groups < kMaxPartials ? groups : kMaxPartials;
        void *args[] = {&K};
        if (hipLaunchKernel(V.fn, dim3((unsigned)nblk), dim3(V.info.waves_per_block * 64), args, 0, stream) !=
            hipSuccess)
            return MI_NORM_ERR_HIP;
    } else {
        {
            const int64_t g = P.rows < kMaxGrid ? P.rows : kMaxGrid;
            void *args[] = {&K};
            if (hipLaunchKernel(rowstats_fn(P.dtype, is_ln(P), V.info.vec), dim3((unsigned)g), dim3(256), args, 0,
                                stream) != hipSuccess)
                return MI_NORM_ERR_HIP;
        }
        // columns per workgroup: its lanes' accesses of one row
        const int64_t chunk = (int64_t)V.info.waves_per_block * 64 * V.info.slots * V.info.vec;
        const int64_t gx = (P.d + chunk - 1) / chunk;
        int64_t nrb = 2048 / gx;
        if (nrb < 1) nrb = 1;
        if (nrb > kMaxPartials) nrb = kMaxPartials;
        if (nrb > P.rows) nrb = P.rows;
        int64_t rows_per_block = (P.rows + nrb - 1) / nrb;
        nrb = (P.rows + rows_per_block - 1) / rows_per_block;
        void *args[] = {&K, &rows_per_block};
        if (hipLaunchKernel(V.fn, dim3((unsigned)gx, (unsigned)nrb), dim3(V.info.waves_per_block * 64), args, 0,
                            stream) !=
            hipSuccess)
            return MI_NORM_ERR_HIP;
        nblk = nrb;
    }
    return pg ? launch_reduce(P, K.part, nblk, stream) : MI_NORM_OK;
}

mi_norm_bwd_problem make_bwd(int op, const float *dy, const float *x, const float *p0, const float *mean,
                             const float *rstd, float *dx, float *dp0, float *dp1, int64_t rows, int64_t d,
                             void *ws, int64_t ws_bytes) {
    mi_norm_bwd_problem P;
    std::memset(&P, 0, sizeof(P));
    P.op = op;
    P.dtype = MI_NORM_F32;
    P.rows = rows;
    P.d = d;
    P.dy = dy;
    P.x = x;
    P.dx = dx;
    P.params0 = p0;
    P.mean = mean;
    P.rstd = rstd;
    P.dparams0 = dp0;
    P.dparams1 = dp1;
    P.workspace = ws;
    P.workspace_bytes = ws_bytes;
    return P;
}

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The address of the scratch array on the current device, looked up once
// per device with that device current; nullptr when it cannot be had.
void *scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" {

mi_norm_status mi_norm_bwd_noalloc(const mi_norm_bwd_problem *p, hipStream_t stream) {
    if (!p || p->workspace || p->workspace_bytes) return MI_NORM_ERR_INVALID;
    const int64_t need = workspace_needed_checked(*p);
    if (need < 0 || need > kScratchBytes) return MI_NORM_ERR_INVALID;
    mi_norm_bwd_problem q = *p;
    q.workspace = scratch_ptr();
    if (!q.workspace) return MI_NORM_ERR_HIP;
    q.workspace_bytes = kScratchBytes;
    return run_bwd(-1, q, stream);
}

int64_t mi_norm_bwd_noalloc_limit(void) { return kScratchBytes; }

int64_t mi_norm_bwd_workspace_size(const mi_norm_bwd_problem *p) {
    return p ? workspace_needed_checked(*p) : -1;
}

mi_norm_status mi_norm_bwd(const mi_norm_bwd_problem *p, hipStream_t stream) {
    return p ? run_bwd(-1, *p, stream) : MI_NORM_ERR_INVALID;
}

mi_norm_status mi_norm_bwd_check(const mi_norm_bwd_problem *p) {
    if (!p) return MI_NORM_ERR_INVALID;
    const mi_norm_status st = validate_bwd(*p);
    if (st != MI_NORM_OK) return st;
    return select_bwd(*p) >= 0 ? MI_NORM_OK : MI_NORM_ERR_INVALID;
}

int mi_norm_bwd_select(const mi_norm_bwd_problem *p) { return p ? select_bwd(*p) : -1; }

int mi_norm_bwd_eligible(int id, const mi_norm_bwd_problem *p) { return (p && eligible_bwd(id, *p)) ? 1 : 0; }

mi_norm_status mi_norm_bwd_variant(int id, const mi_norm_bwd_problem *p, hipStream_t stream) {
    if (!p || !variant(id)) return MI_NORM_ERR_INVALID;
    return run_bwd(id, *p, stream);
}

mi_norm_status mi_layernorm_bwd(const float *dy, const float *x, const float *gamma, const float *mean,
                                const float *rstd, float *dx, float *dgamma, float *dbeta, int64_t rows,
                                int64_t d, void *workspace, int64_t workspace_bytes, hipStream_t stream) {
    return run_bwd(-1, make_bwd(MI_NORM_OP_LAYERNORM, dy, x, gamma, mean, rstd, dx, dgamma, dbeta, rows, d,
                                workspace, workspace_bytes), stream);
}

mi_norm_status mi_rmsnorm_bwd(const float *dy, const float *x, const float *w, const float *rstd, float *dx,
                              float *dw, int64_t rows, int64_t d, void *workspace, int64_t workspace_bytes,
                              hipStream_t stream) {
    return run_bwd(-1, make_bwd(MI_NORM_OP_RMSNORM, dy, x, w, nullptr, rstd, dx, dw, nullptr, rows, d, workspace,
                                workspace_bytes), stream);
}

}  // extern "C"
