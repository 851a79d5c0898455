"""Python face of the C reference oracle (ref_norm.c).

TEST INFRASTRUCTURE ONLY: the float64 CPU definition of LayerNorm and RMSNorm
that the GPU kernels are checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  It imports nothing from the HIP library's package and
the library imports nothing from here.

Functions take and return numpy arrays (float32 in, float32 out, plus the
float64 statistics the pins inspect).  16-bit storage (binary16, bfloat16) is
passed as uint16 bit patterns.  The arithmetic itself lives in the C file;
this module only marshals arguments and chains those C steps.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_LIBS: dict[str, ctypes.CDLL] = {}

_F32P = ctypes.POINTER(ctypes.c_float)
_F64P = ctypes.POINTER(ctypes.c_double)


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    lib.oracle_layernorm_f64.restype = None
    lib.oracle_layernorm_f64.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
    ]
    lib.oracle_rmsnorm_f64.restype = None
    lib.oracle_rmsnorm_f64.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
    ]
    lib.oracle_widen16.restype = ctypes.c_double
    lib.oracle_widen16.argtypes = [ctypes.c_uint16, ctypes.c_int]
    lib.oracle_round16.restype = ctypes.c_uint16
    lib.oracle_round16.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.oracle_widen16_n.restype = None
    lib.oracle_widen16_n.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]
    lib.oracle_round16_n.restype = None
    lib.oracle_round16_n.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]
    lib.oracle_add16_n.restype = None
    lib.oracle_add16_n.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                   ctypes.c_void_p]
    lib.oracle_add_layernorm_f64.restype = None
    lib.oracle_add_layernorm_f64.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
    ]
    lib.oracle_add_rmsnorm_f64.restype = None
    lib.oracle_add_rmsnorm_f64.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
    ]
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.oracle_layernorm_bwd_f64.restype = None
    lib.oracle_layernorm_bwd_f64.argtypes = [vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_rmsnorm_bwd_f64.restype = None
    lib.oracle_rmsnorm_bwd_f64.argtypes = [vp, vp, vp, vp, i64, i64, vp, vp, vp, vp, vp, vp]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_plant.restype = ctypes.c_int
    return lib


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if absent) the oracle library at ``path``."""
    path = path or _build.LIB
    if path not in _LIBS:
        if not os.path.exists(path):
            if path != _build.LIB:
                raise FileNotFoundError(path)
            _build.build()
        _LIBS[path] = _bind(ctypes.CDLL(path))
    return _LIBS[path]


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _f32(a, name: str) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.float32:
        raise TypeError(f"{name} must be float32, got {a.dtype}")
    return np.ascontiguousarray(a)


def layernorm(x, gamma, beta, eps: float = 1e-5, lib: ctypes.CDLL | None = None,
              out: np.ndarray | None = None, y64: np.ndarray | None = None):
    """LayerNorm of each row of ``x`` [rows, d].

    Returns ``(y, mean, rstd, mean64, var64)``: y/mean/rstd rounded once to
    float32, mean64/var64 the float64 statistics before rounding.  ``eps`` is
    taken as the float32 value the GPU receives and widened exactly.  A
    float64 ``y64`` [rows, d] receives the outputs before rounding.
    """
    lib = lib or load()
    x = _f32(x, "x")
    if x.ndim != 2:
        raise ValueError("x must be 2-D [rows, d]")
    rows, d = x.shape
    gamma = _f32(gamma, "gamma").reshape(-1)
    beta = _f32(beta, "beta").reshape(-1)
    if d < 1 or gamma.size != d or beta.size != d:
        raise ValueError("need d >= 1 and gamma, beta of length d")
    y = np.empty_like(x) if out is None else out
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    mean64 = np.empty(rows, np.float64)
    var64 = np.empty(rows, np.float64)
    _check64(y64, x.shape)
    lib.oracle_layernorm_f64(_ptr(x), _ptr(gamma), _ptr(beta), rows, d,
                             float(np.float32(eps)), _ptr(y), _ptr(mean),
                             _ptr(rstd), _ptr(mean64), _ptr(var64), _ptr(y64))
    return y, mean, rstd, mean64, var64


def rmsnorm(x, w, eps: float = 1e-5, lib: ctypes.CDLL | None = None,
            out: np.ndarray | None = None, y64: np.ndarray | None = None):
    """RMSNorm of each row of ``x`` [rows, d].

    Returns ``(y, rstd, ms64)``: y/rstd rounded once to float32, ms64 the
    float64 mean of squares before rounding; ``y64`` as for ``layernorm``.
    """
    lib = lib or load()
    x = _f32(x, "x")
    if x.ndim != 2:
        raise ValueError("x must be 2-D [rows, d]")
    rows, d = x.shape
    w = _f32(w, "w").reshape(-1)
    if d < 1 or w.size != d:
        raise ValueError("need d >= 1 and w of length d")
    y = np.empty_like(x) if out is None else out
    rstd = np.empty(rows, np.float32)
    ms64 = np.empty(rows, np.float64)
    _check64(y64, x.shape)
    lib.oracle_rmsnorm_f64(_ptr(x), _ptr(w), rows, d, float(np.float32(eps)),
                           _ptr(y), _ptr(rstd), _ptr(ms64), _ptr(y64))
    return y, rstd, ms64


def add_layernorm(x, r, gamma, beta, eps: float = 1e-5, lib: ctypes.CDLL | None = None):
    """Residual add then LayerNorm: h = x + r (float32), y = LayerNorm(h).

    Returns ``(y, h, mean, rstd)``.
    """
    lib = lib or load()
    x, r = _f32(x, "x"), _f32(r, "r")
    if x.ndim != 2 or r.shape != x.shape:
        raise ValueError("x and r must be 2-D [rows, d] of one shape")
    rows, d = x.shape
    gamma = _f32(gamma, "gamma").reshape(-1)
    beta = _f32(beta, "beta").reshape(-1)
    if d < 1 or gamma.size != d or beta.size != d:
        raise ValueError("need d >= 1 and gamma, beta of length d")
    y, h = np.empty_like(x), np.empty_like(x)
    mean = np.empty(rows, np.float32)
    rstd = np.empty(rows, np.float32)
    lib.oracle_add_layernorm_f64(_ptr(x), _ptr(r), _ptr(gamma), _ptr(beta), rows, d,
                                 float(np.float32(eps)), _ptr(y), _ptr(h), _ptr(mean), _ptr(rstd))
    return y, h, mean, rstd


def add_rmsnorm(x, r, w, eps: float = 1e-5, lib: ctypes.CDLL | None = None):
    """Residual add then RMSNorm: h = x + r (float32), y = RMSNorm(h).

    Returns ``(y, h, rstd)``.
    """
    lib = lib or load()
    x, r = _f32(x, "x"), _f32(r, "r")
    if x.ndim != 2 or r.shape != x.shape:
        raise ValueError("x and r must be 2-D [rows, d] of one shape")
    rows, d = x.shape
    w = _f32(w, "w").reshape(-1)
    if d < 1 or w.size != d:
        raise ValueError("need d >= 1 and w of length d")
    y, h = np.empty_like(x), np.empty_like(x)
    rstd = np.empty(rows, np.float32)
    lib.oracle_add_rmsnorm_f64(_ptr(x), _ptr(r), _ptr(w), rows, d, float(np.float32(eps)),
                               _ptr(y), _ptr(h), _ptr(rstd))
    return y, h, rstd


# ----------------------------------------------------------------------------
# 16-bit storage: exact widening, one rounding of each float64 output

FMT_F16 = 1   # IEEE binary16
FMT_BF16 = 2  # bfloat16
_FMT_P_EMIN = {FMT_F16: (11, -14), FMT_BF16: (8, -126)}


def _check64(a, shape):
    if a is not None and (a.dtype != np.float64 or a.shape != tuple(shape) or not a.flags.c_contiguous):
        raise ValueError("y64 must be a C-contiguous float64 array of x's shape")


def _u16(a, name: str) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"{name} must hold uint16 bit patterns, got {a.dtype}")
    return np.ascontiguousarray(a)


def widen16(bits, fmt: int, lib: ctypes.CDLL | None = None) -> np.ndarray:
    """float32 values of 16-bit patterns (exact)."""
    lib = lib or load()
    bits = _u16(bits, "bits")
    out = np.empty(bits.shape, np.float32)
    lib.oracle_widen16_n(_ptr(bits), int(fmt), bits.size, _ptr(out))
    return out


def round16(values, fmt: int, lib: ctypes.CDLL | None = None) -> np.ndarray:
    """16-bit patterns nearest (ties to even) to float64 ``values``."""
    lib = lib or load()
    v = np.ascontiguousarray(np.asarray(values, np.float64))
    out = np.empty(v.shape, np.uint16)
    lib.oracle_round16_n(_ptr(v), int(fmt), v.size, _ptr(out))
    return out


def add16(x, r, fmt: int, lib: ctypes.CDLL | None = None) -> np.ndarray:
    """x + r rounded once to the 16-bit format (patterns in, patterns out)."""
    lib = lib or load()
    x, r = _u16(x, "x"), _u16(r, "r")
    if x.shape != r.shape:
        raise ValueError("x and r must have one shape")
    h = np.empty(x.shape, np.uint16)
    lib.oracle_add16_n(_ptr(x), _ptr(r), int(fmt), x.size, _ptr(h))
    return h


def layernorm16(x, fmt: int, gamma, beta, eps: float = 1e-5, lib: ctypes.CDLL | None = None):
    """LayerNorm over 16-bit storage; float32 parameters and statistics.

    Returns ``(y, y64, mean, rstd)``: y the 16-bit patterns of the float64
    outputs ``y64`` rounded once, mean/rstd float32."""
    lib = lib or load()
    xf = widen16(x, fmt, lib)
    y64 = np.empty(xf.shape, np.float64)
    _, mean, rstd, _, _ = layernorm(xf, gamma, beta, eps, lib=lib, y64=y64)
    return round16(y64, fmt, lib), y64, mean, rstd


def rmsnorm16(x, fmt: int, w, eps: float = 1e-5, lib: ctypes.CDLL | None = None):
    """RMSNorm over 16-bit storage; returns ``(y, y64, rstd)``."""
    lib = lib or load()
    xf = widen16(x, fmt, lib)
    y64 = np.empty(xf.shape, np.float64)
    _, rstd, _ = rmsnorm(xf, w, eps, lib=lib, y64=y64)
    return round16(y64, fmt, lib), y64, rstd


def add_layernorm16(x, r, fmt: int, gamma, beta, eps: float = 1e-5, lib: ctypes.CDLL | None = None):
    """Residual add in the storage format, then LayerNorm of that stored sum.

    Returns ``(y, y64, h, mean, rstd)``."""
    lib = lib or load()
    h = add16(x, r, fmt, lib)
    y, y64, mean, rstd = layernorm16(h, fmt, gamma, beta, eps, lib)
    return y, y64, h, mean, rstd


def add_rmsnorm16(x, r, fmt: int, w, eps: float = 1e-5, lib: ctypes.CDLL | None = None):
    """Residual add in the storage format, then RMSNorm; ``(y, y64, h, rstd)``."""
    lib = lib or load()
    h = add16(x, r, fmt, lib)
    y, y64, rstd = rmsnorm16(h, fmt, w, eps, lib)
    return y, y64, h, rstd


def ulp16(mag, fmt: int) -> np.ndarray:
    """The spacing of the 16-bit format at magnitude ``mag`` (the subnormal
    spacing below the normal range)."""
    p, emin = _FMT_P_EMIN[fmt]
    m = np.abs(np.asarray(mag, np.float64))
    _, e = np.frexp(m)                        # m = f * 2^e, 0.5 <= f < 1
    E = np.maximum(e.astype(np.int64) - 1, emin)
    return np.ldexp(1.0, (E - (p - 1)).astype(np.int64))


def tolerance_ok16(got_bits, ref64, fmt: int, atol: float = 1e-5, rtol: float = 1e-4,
                   lib: ctypes.CDLL | None = None):
    """Acceptance for outputs stored in a 16-bit format.

    A kernel that meets the float32 bound tau = atol + rtol*|ref| before its
    final rounding, then rounds to nearest, lands within tau plus half a
    16-bit ulp of the exact value; the ulp is taken at the larger of |got| and
    |ref| + tau, which covers a rounding across a power of two.  Returns
    ``(ok, max_abs_err, max_ratio)`` like ``tolerance_ok``."""
    got = widen16(got_bits, fmt, lib).astype(np.float64)
    ref = np.asarray(ref64, np.float64)
    if got.shape != ref.shape:
        return False, float("inf"), float("inf")
    if got.size == 0:
        return True, 0.0, 0.0
    if not np.all(np.isfinite(got)) or not np.all(np.isfinite(ref)):
        return False, float("inf"), float("inf")
    tau = atol + rtol * np.abs(ref)
    bound = tau + 0.5 * ulp16(np.maximum(np.abs(got), np.abs(ref) + tau), fmt)
    err = np.abs(got - ref)
    ratio = err / bound
    return bool(np.all(err <= bound)), float(err.max()), float(ratio.max())


# ----------------------------------------------------------------------------
# backward: gradients with respect to x and the per-column parameters

def _stats64(a, rows: int, name: str) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(a, np.float64).reshape(-1))
    if a.size != rows:
        raise ValueError(f"{name} must hold one value per row")
    return a


def layernorm_bwd(dy, x, gamma, mean, rstd, lib: ctypes.CDLL | None = None) -> dict:
    """LayerNorm backward from the upstream gradient dy and the forward's
    per-row statistics (float32 or float64; widened exactly).

    Returns a dict: dx (float32) and dx64, dx_scale (per element, the
    magnitudes a float32 evaluation of dx carries error in proportion to),
    dgamma/dbeta (float32) and dgamma64/dbeta64, and abs_dgamma/abs_dbeta
    (sum over rows of |dy xhat| and |dy|, the magnitudes a float32 column
    sum's error scales with)."""
    lib = lib or load()
    dy, x = _f32(dy, "dy"), _f32(x, "x")
    if x.ndim != 2 or dy.shape != x.shape:
        raise ValueError("dy and x must be 2-D [rows, d] of one shape")
    rows, d = x.shape
    gamma = _f32(gamma, "gamma").reshape(-1)
    if d < 1 or gamma.size != d:
        raise ValueError("need d >= 1 and gamma of length d")
    m64, r64 = _stats64(mean, rows, "mean"), _stats64(rstd, rows, "rstd")
    out = dict(dx=np.empty_like(x), dx64=np.empty(x.shape, np.float64), dx_scale=np.empty(x.shape, np.float64),
               dgamma=np.empty(d, np.float32), dbeta=np.empty(d, np.float32),
               dgamma64=np.empty(d), dbeta64=np.empty(d), abs_dgamma=np.empty(d), abs_dbeta=np.empty(d))
    lib.oracle_layernorm_bwd_f64(_ptr(dy), _ptr(x), _ptr(gamma), _ptr(m64), _ptr(r64), rows, d,
                                 _ptr(out["dx"]), _ptr(out["dx64"]), _ptr(out["dx_scale"]),
                                 _ptr(out["dgamma"]), _ptr(out["dbeta"]),
                                 _ptr(out["dgamma64"]), _ptr(out["dbeta64"]), _ptr(out["abs_dgamma"]),
                                 _ptr(out["abs_dbeta"]))
    return out


def rmsnorm_bwd(dy, x, w, rstd, lib: ctypes.CDLL | None = None) -> dict:
    """RMSNorm backward; dict with dx, dx64, dx_scale, dw, dw64, abs_dw."""
    lib = lib or load()
    dy, x = _f32(dy, "dy"), _f32(x, "x")
    if x.ndim != 2 or dy.shape != x.shape:
        raise ValueError("dy and x must be 2-D [rows, d] of one shape")
    rows, d = x.shape
    w = _f32(w, "w").reshape(-1)
    if d < 1 or w.size != d:
        raise ValueError("need d >= 1 and w of length d")
    r64 = _stats64(rstd, rows, "rstd")
    out = dict(dx=np.empty_like(x), dx64=np.empty(x.shape, np.float64), dx_scale=np.empty(x.shape, np.float64),
               dw=np.empty(d, np.float32), dw64=np.empty(d), abs_dw=np.empty(d))
    lib.oracle_rmsnorm_bwd_f64(_ptr(dy), _ptr(x), _ptr(w), _ptr(r64), rows, d, _ptr(out["dx"]),
                               _ptr(out["dx64"]), _ptr(out["dx_scale"]), _ptr(out["dw"]), _ptr(out["dw64"]),
                               _ptr(out["abs_dw"]))
    return out


def layernorm_bwd16(dy, x, fmt: int, gamma, mean, rstd, lib: ctypes.CDLL | None = None) -> dict:
    """LayerNorm backward over 16-bit dy and x (patterns); adds dx16, dx
    rounded once to the format from dx64.  Parameter gradients stay float32."""
    lib = lib or load()
    out = layernorm_bwd(widen16(dy, fmt, lib), widen16(x, fmt, lib), gamma, mean, rstd, lib)
    out["dx16"] = round16(out["dx64"], fmt, lib)
    return out


def rmsnorm_bwd16(dy, x, fmt: int, w, rstd, lib: ctypes.CDLL | None = None) -> dict:
    lib = lib or load()
    out = rmsnorm_bwd(widen16(dy, fmt, lib), widen16(x, fmt, lib), w, rstd, lib)
    out["dx16"] = round16(out["dx64"], fmt, lib)
    return out


U32 = 2.0 ** -24  # unit roundoff of float32


def colsum_tolerance_ok(got, ref64, abs_sum, atol: float = 1e-5, rtol: float = 1e-4, k: float = 6.0):
    """Acceptance for a float32 sum over rows (the parameter gradients).

    The float32 bound of the forward outputs plus k * u * sum|terms|, for any
    evaluation that forms each term in float32 from the float32 inputs,
    carries every sum in float64, and rounds to float32 only partial sums
    over subsets of the rows, at most two nested levels of them (each
    partial once), and the final sum: each term dy * xhat carries at most
    three float32 roundings (x - mean, times rstd, times dy: <= 3u of
    |term|); each level of partial sums adds <= u * sum|terms| whatever the
    partition; a float64 sum of n terms in any order errs by
    <= n 2^-53 sum|terms|, which is <= u * sum|terms| for up to 2^29 rows;
    the final rounding is inside rtol.  That is k = 6, whatever the order of
    the additions or the split of the rows into partial sums.
    Returns ``(ok, max_abs_err, max_ratio)``."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref64, np.float64)
    a = np.asarray(abs_sum, np.float64)
    if got.shape != ref.shape or a.shape != ref.shape:
        return False, float("inf"), float("inf")
    if got.size == 0:
        return True, 0.0, 0.0
    if not np.all(np.isfinite(got)):
        return False, float("inf"), float("inf")
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref) + k * U32 * a
    return bool(np.all(err <= bound)), float(err.max()), float((err / bound).max())


def dx_tolerance_ok(got, ref64, scale64, fmt: int | None = None, atol: float = 1e-5, rtol: float = 1e-4,
                    k: float = 16.0, lib: ctypes.CDLL | None = None):
    """Acceptance for dx: the float32 bound plus k * u * scale (and, for a
    16-bit dx given as patterns with ``fmt``, half a 16-bit ulp).

    dx = rstd * (g - mean(g) - xhat * mean(g xhat)) subtracts quantities of
    the size of |g|, mean|g| and |xhat| mean|g xhat| (``dx_scale`` holds
    rstd times their sum).  Consider any evaluation that forms g, xhat and
    g xhat in float32 from the float32 inputs, adds a row's terms in float32
    only within groups of at most eight (a pairwise sum: three roundings),
    carries the rest of the row sum in float64 in any order and rounds each
    mean once to float32.  Its errors, in units of u and to first order:
    g 1, xhat 2; mean(g) 5 of mean|g| (its terms' rounding, the group's
    three, its own); mean(g xhat) 8 of mean|g xhat| (four for the terms,
    three, one); xhat * mean(g xhat) 11 of |xhat| mean|g xhat|; then the two
    subtractions and the product with rstd, one each of the whole scale.  The
    sum is <= 14 u * scale (the float64 sums add d 2^-53, nothing at these
    widths); k = 16.  When rstd is large (a row of near-zero variance gives
    ~1/sqrt(eps)), these errors are far above the float32 bound of the
    forward outputs while the exact dx may be ~0, which is why the bound
    scales with rstd.  Returns ``(ok, max_abs_err, max_ratio)``."""
    ref = np.asarray(ref64, np.float64)
    if fmt is None:
        got = np.asarray(got, np.float64)
    else:
        got = widen16(got, fmt, lib).astype(np.float64)
    s = np.asarray(scale64, np.float64)
    if got.shape != ref.shape or s.shape != ref.shape:
        return False, float("inf"), float("inf")
    if got.size == 0:
        return True, 0.0, 0.0
    if not np.all(np.isfinite(got)):
        return False, float("inf"), float("inf")
    tau = atol + rtol * np.abs(ref) + k * U32 * s
    bound = tau if fmt is None else tau + 0.5 * ulp16(np.maximum(np.abs(got), np.abs(ref) + tau), fmt)
    err = np.abs(got - ref)
    return bool(np.all(err <= bound)), float(err.max()), float((err / bound).max())


def set_threads(n: int, lib: ctypes.CDLL | None = None) -> None:
    (lib or load()).oracle_set_threads(int(n))


def max_threads(lib: ctypes.CDLL | None = None) -> int:
    return int((lib or load()).oracle_max_threads())


def tolerance_ok(got, ref, atol: float = 1e-5, rtol: float = 1e-4):
    """Elementwise acceptance used throughout: |got - ref| <= atol + rtol*|ref|.

    The bound is the one stated on "RMSNorm on an RTX 5070" (section
    "Correctness before timing").  Any NaN/Inf in ``got`` fails.  Returns
    ``(ok, max_abs_err, max_ratio)`` where max_ratio is the worst
    err / bound.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        return False, float("inf"), float("inf")
    if got.size == 0:
        return True, 0.0, 0.0
    if not np.all(np.isfinite(got)) or not np.all(np.isfinite(ref)):
        return False, float("inf"), float("inf")
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    ratio = err / bound
    return bool(np.all(err <= bound)), float(err.max()), float(ratio.max())
