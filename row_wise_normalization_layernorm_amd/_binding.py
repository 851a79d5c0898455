"""ctypes binding of libmi_norm.so (include/mi_norm.h, and the tuning and
calibration calls of include/mi_norm_tuning.h).

Argument marshalling only: every arithmetic step runs in the library's HIP
kernels.  Functions accept torch CUDA tensors (their device pointer is taken)
or plain integers (raw device addresses).  ``stream`` may be None (torch's
current stream of the tensors' device, else the null stream), an int handle,
or a ``torch.cuda.Stream``.

torch is imported before the library is loaded: the library's HIP runtime
dependency (SONAME libamdhip64.so.7) then resolves to the runtime torch has
already mapped, so torch's streams and allocations are valid inside it.  If
the library has not been built, every call raises RuntimeError; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmi_norm.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "mi_norm.h")
TUNING_HEADER = os.path.join(os.path.dirname(PKG), "include", "mi_norm_tuning.h")

MI_NORM_OK = 0
MI_NORM_ERR_INVALID = 1
MI_NORM_ERR_HIP = 2
OP_LAYERNORM = 0
OP_RMSNORM = 1
OP_ADD_LAYERNORM = 2
OP_ADD_RMSNORM = 3
OP_LAYERNORM_BWD = 4
OP_RMSNORM_BWD = 5
MI_NORM_F32 = 0
MI_NORM_F16 = 1
MI_NORM_BF16 = 2

_lib = None


class MiNormError(RuntimeError):
    """A non-OK status from the C ABI; ``.status`` holds the code."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class VariantInfo(ctypes.Structure):
    _fields_ = [
        ("op", ctypes.c_int), ("dtype", ctypes.c_int), ("vec", ctypes.c_int), ("peel", ctypes.c_int),
        ("looped", ctypes.c_int), ("lanes_per_row", ctypes.c_int),
        ("waves_per_row", ctypes.c_int), ("slots", ctypes.c_int),
        ("waves_per_block", ctypes.c_int), ("rows_per_block", ctypes.c_int),
        ("max_d", ctypes.c_int64), ("needs_aligned", ctypes.c_int), ("rows_per_lane", ctypes.c_int),
    ]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}


class Problem(ctypes.Structure):
    """mi_norm_problem: one call in full (mi_norm_fwd, the variant queries)."""
    _fields_ = [
        ("op", ctypes.c_int), ("dtype", ctypes.c_int), ("rows", ctypes.c_int64), ("d", ctypes.c_int64),
        ("x", ctypes.c_void_p), ("ldx", ctypes.c_int64), ("r", ctypes.c_void_p), ("ldr", ctypes.c_int64),
        ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64), ("h", ctypes.c_void_p), ("ldh", ctypes.c_int64),
        ("params0", ctypes.c_void_p), ("params1", ctypes.c_void_p), ("eps", ctypes.c_float),
        ("mean", ctypes.c_void_p), ("rstd", ctypes.c_void_p),
    ]


class BwdProblem(ctypes.Structure):
    """mi_norm_bwd_problem: one backward call in full."""
    _fields_ = [
        ("op", ctypes.c_int), ("dtype", ctypes.c_int), ("rows", ctypes.c_int64), ("d", ctypes.c_int64),
        ("dy", ctypes.c_void_p), ("lddy", ctypes.c_int64), ("x", ctypes.c_void_p), ("ldx", ctypes.c_int64),
        ("dx", ctypes.c_void_p), ("lddx", ctypes.c_int64), ("params0", ctypes.c_void_p),
        ("mean", ctypes.c_void_p), ("rstd", ctypes.c_void_p), ("dparams0", ctypes.c_void_p),
        ("dparams1", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
    ]


_VP = ctypes.c_void_p
_I64 = ctypes.c_int64
_F = ctypes.c_float
_I = ctypes.c_int

_SIGNATURES = {
    "mi_norm_status_string": (ctypes.c_char_p, [_I]),
    "mi_norm_version": (ctypes.c_char_p, []),
    "mi_layernorm_fwd": (_I, [_VP, _VP, _VP, _VP, _I64, _I64, _F, _VP, _VP, _VP]),
    "mi_rmsnorm_fwd": (_I, [_VP, _VP, _VP, _I64, _I64, _F, _VP, _VP]),
    "mi_norm_variant_count": (_I, []),
    "mi_norm_variant_name": (ctypes.c_char_p, [_I]),
    "mi_norm_variant_get_info": (_I, [_I, ctypes.POINTER(VariantInfo)]),
    "mi_add_layernorm_fwd": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _F, _VP, _VP, _VP]),
    "mi_add_rmsnorm_fwd": (_I, [_VP, _VP, _VP, _VP, _VP, _I64, _I64, _F, _VP, _VP]),
    "mi_norm_fwd": (_I, [ctypes.POINTER(Problem), _VP]),
    "mi_norm_fwd_variant": (_I, [_I, ctypes.POINTER(Problem), _VP]),
    "mi_norm_check": (_I, [ctypes.POINTER(Problem)]),
    "mi_norm_select": (_I, [ctypes.POINTER(Problem)]),
    "mi_norm_eligible": (_I, [_I, ctypes.POINTER(Problem)]),
    "mi_add_layernorm_fwd_variant": (_I, [_I, _VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _F, _VP, _VP,
                                          _VP]),
    "mi_add_rmsnorm_fwd_variant": (_I, [_I, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _F, _VP, _VP]),
    "mi_layernorm_fwd_variant": (_I, [_I, _VP, _VP, _VP, _VP, _I64, _I64, _F, _VP, _VP, _VP]),
    "mi_rmsnorm_fwd_variant": (_I, [_I, _VP, _VP, _VP, _I64, _I64, _F, _VP, _VP]),
    "mi_copy_f32": (_I, [_VP, _VP, _I64, _VP]),
    "mi_calib_launch": (_I, [_I, _VP, _VP, _I64, _VP]),
    "mi_norm_bwd_workspace_size": (_I64, [ctypes.POINTER(BwdProblem)]),
    "mi_norm_bwd": (_I, [ctypes.POINTER(BwdProblem), _VP]),
    "mi_norm_bwd_noalloc": (_I, [ctypes.POINTER(BwdProblem), _VP]),
    "mi_norm_bwd_noalloc_limit": (_I64, []),
    "mi_norm_bwd_check": (_I, [ctypes.POINTER(BwdProblem)]),
    "mi_norm_bwd_select": (_I, [ctypes.POINTER(BwdProblem)]),
    "mi_norm_bwd_eligible": (_I, [_I, ctypes.POINTER(BwdProblem)]),
    "mi_norm_bwd_variant": (_I, [_I, ctypes.POINTER(BwdProblem), _VP]),
    "mi_layernorm_bwd": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _VP, _I64, _VP]),
    "mi_rmsnorm_bwd": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _VP, _I64, _VP]),
}


def header_functions(path: str | None = None) -> list[str]:
    """Names of the functions a header declares: include/mi_norm.h and
    include/mi_norm_tuning.h together by default."""
    names = set()
    for p in ([path] if path else [HEADER, TUNING_HEADER]):
        text = re.sub(r"/\*.*?\*/", "", open(p).read(), flags=re.S)
        names |= set(re.findall(r"\b(mi_\w+)\s*\(", text))
    return sorted(names)


def lib() -> ctypes.CDLL:
    """The loaded library (loading it on first use)."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (see module docstring: runtime order)
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(python -m row_wise_normalization_layernorm_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != MI_NORM_OK:
        msg = lib().mi_norm_status_string(status).decode()
        raise MiNormError(status, f"{what}: {msg}")


def _is_tensor(a) -> bool:
    return type(a).__module__.startswith("torch") and hasattr(a, "data_ptr")


def _ptr(a, name: str, need: int | None = None):
    """Device address of a tensor (validated) or an int; None stays None."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if _is_tensor(a):
        import torch
        if a.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor, got {a.device}")
        if a.dtype != torch.float32:
            raise ValueError(f"{name} must be float32, got {a.dtype}")
        if not a.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if need is not None and a.numel() < need:
            raise ValueError(f"{name} holds {a.numel()} elements, needs {need}")
        return a.data_ptr()
    raise TypeError(f"{name}: expected a torch tensor, an int address or None")


def _stream(stream, *tensors):
    if stream is None:
        for t in tensors:
            if t is not None and _is_tensor(t) and t.device.type == "cuda":
                import torch
                return torch.cuda.current_stream(t.device).cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# --- the C entry points, same names -----------------------------------------

def mi_layernorm_fwd(x, gamma, beta, y, rows: int, d: int, eps: float = 1e-5,
                     mean=None, rstd=None, stream=None) -> None:
    n = max(rows, 0) * max(d, 0)
    st = lib().mi_layernorm_fwd(_ptr(x, "x", n), _ptr(gamma, "gamma", d), _ptr(beta, "beta", d),
                                _ptr(y, "y", n), rows, d, eps, _ptr(mean, "mean", rows),
                                _ptr(rstd, "rstd", rows), _stream(stream, x, y))
    _check(st, "mi_layernorm_fwd")


def mi_rmsnorm_fwd(x, w, y, rows: int, d: int, eps: float = 1e-5, rstd=None,
                   stream=None) -> None:
    n = max(rows, 0) * max(d, 0)
    st = lib().mi_rmsnorm_fwd(_ptr(x, "x", n), _ptr(w, "w", d), _ptr(y, "y", n), rows, d, eps,
                              _ptr(rstd, "rstd", rows), _stream(stream, x, y))
    _check(st, "mi_rmsnorm_fwd")


def mi_layernorm_fwd_variant(vid: int, x, gamma, beta, y, rows: int, d: int, eps: float = 1e-5,
                             mean=None, rstd=None, stream=None) -> None:
    n = max(rows, 0) * max(d, 0)
    st = lib().mi_layernorm_fwd_variant(vid, _ptr(x, "x", n), _ptr(gamma, "gamma", d),
                                        _ptr(beta, "beta", d), _ptr(y, "y", n), rows, d, eps,
                                        _ptr(mean, "mean", rows), _ptr(rstd, "rstd", rows),
                                        _stream(stream, x, y))
    _check(st, f"mi_layernorm_fwd_variant({vid})")


def mi_rmsnorm_fwd_variant(vid: int, x, w, y, rows: int, d: int, eps: float = 1e-5, rstd=None,
                           stream=None) -> None:
    n = max(rows, 0) * max(d, 0)
    st = lib().mi_rmsnorm_fwd_variant(vid, _ptr(x, "x", n), _ptr(w, "w", d), _ptr(y, "y", n),
                                      rows, d, eps, _ptr(rstd, "rstd", rows), _stream(stream, x, y))
    _check(st, f"mi_rmsnorm_fwd_variant({vid})")


def mi_add_layernorm_fwd(x, r, gamma, beta, y, h, rows: int, d: int, eps: float = 1e-5,
                         mean=None, rstd=None, stream=None) -> None:
    n = max(rows, 0) * max(d, 0)
    st = lib().mi_add_layernorm_fwd(_ptr(x, "x", n), _ptr(r, "r", n), _ptr(gamma, "gamma", d),
                                    _ptr(beta, "beta", d), _ptr(y, "y", n), _ptr(h, "h", n), rows, d,
                                    eps, _ptr(mean, "mean", rows), _ptr(rstd, "rstd", rows),
                                    _stream(stream, x, y))
    _check(st, "mi_add_layernorm_fwd")


def mi_add_rmsnorm_fwd(x, r, w, y, h, rows: int, d: int, eps: float = 1e-5, rstd=None,
                       stream=None) -> None:
    n = max(rows, 0) * max(d, 0)
    st = lib().mi_add_rmsnorm_fwd(_ptr(x, "x", n), _ptr(r, "r", n), _ptr(w, "w", d), _ptr(y, "y", n),
                                  _ptr(h, "h", n), rows, d, eps, _ptr(rstd, "rstd", rows),
                                  _stream(stream, x, y))
    _check(st, "mi_add_rmsnorm_fwd")


def mi_add_layernorm_fwd_variant(vid: int, x, r, gamma, beta, y, h, rows: int, d: int,
                                 eps: float = 1e-5, mean=None, rstd=None, stream=None) -> None:
    n = max(rows, 0) * max(d, 0)
    st = lib().mi_add_layernorm_fwd_variant(vid, _ptr(x, "x", n), _ptr(r, "r", n),
                                            _ptr(gamma, "gamma", d), _ptr(beta, "beta", d),
                                            _ptr(y, "y", n), _ptr(h, "h", n), rows, d, eps,
                                            _ptr(mean, "mean", rows), _ptr(rstd, "rstd", rows),
                                            _stream(stream, x, y))
    _check(st, f"mi_add_layernorm_fwd_variant({vid})")


def mi_add_rmsnorm_fwd_variant(vid: int, x, r, w, y, h, rows: int, d: int, eps: float = 1e-5,
                               rstd=None, stream=None) -> None:
    n = max(rows, 0) * max(d, 0)
    st = lib().mi_add_rmsnorm_fwd_variant(vid, _ptr(x, "x", n), _ptr(r, "r", n), _ptr(w, "w", d),
                                          _ptr(y, "y", n), _ptr(h, "h", n), rows, d, eps,
                                          _ptr(rstd, "rstd", rows), _stream(stream, x, y))
    _check(st, f"mi_add_rmsnorm_fwd_variant({vid})")


def mi_copy_f32(src, dst, n: int, stream=None) -> None:
    st = lib().mi_copy_f32(_ptr(src, "src", n), _ptr(dst, "dst", n), n, _stream(stream, src, dst))
    _check(st, "mi_copy_f32")


def mi_calib_launch(kind: int, src, dst, n: int, stream=None) -> None:
    """A calibration launch (mi_norm_tuning.h): kind 0 empty, 1 read n float32
    from src, 2 write n float32 to dst."""
    st = lib().mi_calib_launch(kind, _ptr(src, "src", n if kind == 1 else None),
                               _ptr(dst, "dst", n if kind == 2 else None), n, _stream(stream, src, dst))
    _check(st, "mi_calib_launch")


def mi_norm_status_string(status: int) -> str:
    return lib().mi_norm_status_string(status).decode()


def mi_norm_version() -> str:
    return lib().mi_norm_version().decode()


def mi_norm_variant_count() -> int:
    return int(lib().mi_norm_variant_count())


def mi_norm_variant_name(vid: int) -> str | None:
    r = lib().mi_norm_variant_name(vid)
    return None if r is None else r.decode()


def mi_norm_variant_get_info(vid: int) -> dict:
    info = VariantInfo()
    _check(lib().mi_norm_variant_get_info(vid, ctypes.byref(info)), "mi_norm_variant_get_info")
    return info.as_dict()


def _addr(a):
    return a if (a is None or isinstance(a, int)) else a.data_ptr()


def problem(op: int, rows: int, d: int, x, y, params0, params1=None, r=None, h=None, *,
            dtype: int = MI_NORM_F32, ldx: int = 0, ldr: int = 0, ldy: int = 0, ldh: int = 0,
            eps: float = 1e-5, mean=None, rstd=None) -> Problem:
    """An mi_norm_problem from tensors or integer addresses (strides in
    elements, 0 meaning d)."""
    return Problem(op, dtype, rows, d, _addr(x), ldx, _addr(r), ldr, _addr(y), ldy, _addr(h), ldh,
                   _addr(params0), _addr(params1), eps, _addr(mean), _addr(rstd))


def mi_norm_fwd(p: Problem, stream=None) -> None:
    _check(lib().mi_norm_fwd(ctypes.byref(p), _stream(stream)), "mi_norm_fwd")


def mi_norm_check(p: Problem) -> int:
    """Status mi_norm_fwd would return before launching (host logic only)."""
    return int(lib().mi_norm_check(ctypes.byref(p)))


def mi_norm_fwd_variant(vid: int, p: Problem, stream=None) -> None:
    _check(lib().mi_norm_fwd_variant(vid, ctypes.byref(p), _stream(stream)), f"mi_norm_fwd_variant({vid})")


def mi_norm_select(p: Problem) -> int:
    return int(lib().mi_norm_select(ctypes.byref(p)))


def mi_norm_eligible(vid: int, p: Problem) -> bool:
    return bool(lib().mi_norm_eligible(vid, ctypes.byref(p)))


def bwd_problem(op: int, rows: int, d: int, dy, x, dx, params0, mean=None, rstd=None, dparams0=None,
                dparams1=None, workspace=None, workspace_bytes: int = 0, *, dtype: int = MI_NORM_F32,
                lddy: int = 0, ldx: int = 0, lddx: int = 0) -> BwdProblem:
    """An mi_norm_bwd_problem (op OP_LAYERNORM or OP_RMSNORM) from tensors or
    integer addresses."""
    return BwdProblem(op, dtype, rows, d, _addr(dy), lddy, _addr(x), ldx, _addr(dx), lddx, _addr(params0),
                      _addr(mean), _addr(rstd), _addr(dparams0), _addr(dparams1), _addr(workspace),
                      workspace_bytes)


def mi_norm_bwd_workspace_size(p: BwdProblem) -> int:
    return int(lib().mi_norm_bwd_workspace_size(ctypes.byref(p)))


def mi_norm_bwd(p: BwdProblem, stream=None) -> None:
    _check(lib().mi_norm_bwd(ctypes.byref(p), _stream(stream)), "mi_norm_bwd")


def mi_norm_bwd_noalloc(p: BwdProblem, stream=None) -> None:
    """mi_norm_bwd with the library's own scratch array as the workspace
    (p.workspace None, p.workspace_bytes 0); allocates nothing."""
    _check(lib().mi_norm_bwd_noalloc(ctypes.byref(p), _stream(stream)), "mi_norm_bwd_noalloc")


def mi_norm_bwd_noalloc_limit() -> int:
    return int(lib().mi_norm_bwd_noalloc_limit())


def mi_norm_bwd_check(p: BwdProblem) -> int:
    return int(lib().mi_norm_bwd_check(ctypes.byref(p)))


def mi_norm_bwd_select(p: BwdProblem) -> int:
    return int(lib().mi_norm_bwd_select(ctypes.byref(p)))


def mi_norm_bwd_eligible(vid: int, p: BwdProblem) -> bool:
    return bool(lib().mi_norm_bwd_eligible(vid, ctypes.byref(p)))


def mi_norm_bwd_variant(vid: int, p: BwdProblem, stream=None) -> None:
    _check(lib().mi_norm_bwd_variant(vid, ctypes.byref(p), _stream(stream)), f"mi_norm_bwd_variant({vid})")


def mi_layernorm_bwd(dy, x, gamma, mean, rstd, dx, dgamma, dbeta, rows: int, d: int, workspace,
                     workspace_bytes: int, stream=None) -> None:
    n = max(rows, 0) * max(d, 0)
    st = lib().mi_layernorm_bwd(_ptr(dy, "dy", n), _ptr(x, "x", n), _ptr(gamma, "gamma", d),
                                _ptr(mean, "mean", rows), _ptr(rstd, "rstd", rows), _ptr(dx, "dx", n),
                                _ptr(dgamma, "dgamma", d), _ptr(dbeta, "dbeta", d), rows, d,
                                _addr(workspace), workspace_bytes, _stream(stream, dy, dx))
    _check(st, "mi_layernorm_bwd")


def mi_rmsnorm_bwd(dy, x, w, rstd, dx, dw, rows: int, d: int, workspace, workspace_bytes: int,
                   stream=None) -> None:
    n = max(rows, 0) * max(d, 0)
    st = lib().mi_rmsnorm_bwd(_ptr(dy, "dy", n), _ptr(x, "x", n), _ptr(w, "w", d), _ptr(rstd, "rstd", rows),
                              _ptr(dx, "dx", n), _ptr(dw, "dw", d), rows, d, _addr(workspace), workspace_bytes,
                              _stream(stream, dy, dx))
    _check(st, "mi_rmsnorm_bwd")


# --- conveniences over torch tensors (allocation is torch's) -------------------

def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: MI_NORM_F32, torch.float16: MI_NORM_F16, torch.bfloat16: MI_NORM_BF16}
    if t.dtype not in codes:
        raise ValueError(f"rows must be float32, float16 or bfloat16, got {t.dtype}")
    return codes[t.dtype]


def _row_geometry(shape, strides, name: str) -> tuple[int, int]:
    """(rows, row stride in elements) of a tensor of ``shape``/``strides``
    [..., d] whose last dimension is contiguous and whose leading dimensions
    form one strided row index.  Rows that repeat one another (a leading
    dimension expanded with stride 0) are refused: the C ABI reads a row
    stride of 0 as d, so such rows would be addressed past the tensor's
    storage."""
    if len(shape) == 0:
        raise ValueError(f"{name} must have a last dimension")
    d = shape[-1]
    if d > 1 and strides[-1] != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    if len(shape) == 1:
        return 1, d
    lead = [(s, st) for s, st in zip(shape[:-1], strides[:-1]) if s != 1]
    rows = 1
    for s, _ in lead:
        rows *= s
    if not lead:
        return rows, d
    if any(st == 0 for _, st in lead):
        raise ValueError(f"{name}: rows repeat one another (a leading dimension has stride 0)")
    for (s0, st0), (s1, st1) in zip(lead, lead[1:]):
        if st0 != st1 * s1:
            raise ValueError(f"{name}: leading dimensions do not form one row stride")
    return rows, lead[-1][1]


def _rows_of(t, name: str) -> tuple[int, int]:
    """(rows, row stride in elements) of a device row tensor; no copy is made."""
    if not _is_tensor(t) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    return _row_geometry(tuple(t.shape), tuple(t.stride()), name)


def _input_rows(t):
    """An input row tensor as the kernels can read it: one whose rows repeat
    one another (stride 0, e.g. the upstream gradient of a sum over rows)
    is made contiguous; anything else is passed as it is."""
    if _is_tensor(t) and t.dim() > 1 and any(s != 1 and st == 0 for s, st in zip(t.shape[:-1], t.stride()[:-1])):
        return t.contiguous()
    return t


def _params(t, name: str, d: int):
    import torch
    if t is None:
        return None
    if not _is_tensor(t) or t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != d:
        raise ValueError(f"{name} must be a contiguous float32 device tensor of {d} elements")
    return t


def _on_stream(stream, device):
    """(context, handle): inside the context, torch allocations belong to the
    stream the kernels will run on, so the caching allocator does not hand
    them to other streams' work before those kernels finish; handle is that
    stream's hipStream_t.  ``stream`` is None (torch's current stream), a
    torch stream, or a raw handle."""
    import contextlib
    import torch
    if stream is None:
        return contextlib.nullcontext(), torch.cuda.current_stream(device).cuda_stream
    if hasattr(stream, "cuda_stream"):
        return torch.cuda.stream(stream), stream.cuda_stream
    return torch.cuda.stream(torch.cuda.ExternalStream(stream, device=device)), stream


def _norm(op, x, r, p0, p1, eps, stats, out, write_sum, stream):
    import torch
    dt = _dtype_code(x)
    d = x.shape[-1]
    if out is not None:
        _rows_of(out, "out")   # an output is never copied: refuse repeating rows before any copy
    x, r = _input_rows(x), _input_rows(r)
    rows, ldx = _rows_of(x, "x")
    ldr = 0
    if r is not None:
        if r.dtype != x.dtype or r.shape != x.shape:
            raise ValueError("r must have x's shape and dtype")
        ldr = _rows_of(r, "r")[1]
    ctx, handle = _on_stream(stream, x.device)
    with ctx:
        y = torch.empty(x.shape, device=x.device, dtype=x.dtype) if out is None else out
        if y.dtype != x.dtype or y.shape != x.shape:
            raise ValueError("out must have x's shape and dtype")
        ldy = _rows_of(y, "out")[1]
        h = torch.empty(x.shape, device=x.device, dtype=x.dtype) if (r is not None and write_sum) else None
        ln = op in (OP_LAYERNORM, OP_ADD_LAYERNORM)
        mean = torch.empty(x.shape[:-1], device=x.device, dtype=torch.float32) if (stats and ln) else None
        rstd = torch.empty(x.shape[:-1], device=x.device, dtype=torch.float32) if stats else None
        p = problem(op, rows, d, x, y, _params(p0, "gamma" if ln else "w", d), _params(p1, "beta", d), r, h,
                    dtype=dt, ldx=ldx, ldr=ldr, ldy=ldy, ldh=0, eps=eps, mean=mean, rstd=rstd)
        mi_norm_fwd(p, handle)
    return y, h, mean, rstd


def layernorm(x, gamma, beta, eps: float = 1e-5, stats: bool = False, out=None, stream=None):
    """LayerNorm over the last dimension of a float32, float16 or bfloat16
    device tensor (rows may be strided; gamma/beta float32).

    Returns y, or (y, mean, rstd) with ``stats``.  ``out`` may be x (in place).
    """
    y, _, mean, rstd = _norm(OP_LAYERNORM, x, None, gamma, beta, eps, stats, out, False, stream)
    return (y, mean, rstd) if stats else y


def add_layernorm(x, r, gamma, beta, eps: float = 1e-5, stats: bool = False, write_sum: bool = True,
                  stream=None):
    """h = x + r, y = LayerNorm(h).  Returns (y, h) or (y, h, mean, rstd); h is
    None without ``write_sum``."""
    y, h, mean, rstd = _norm(OP_ADD_LAYERNORM, x, r, gamma, beta, eps, stats, None, write_sum, stream)
    return (y, h, mean, rstd) if stats else (y, h)


def add_rmsnorm(x, r, w, eps: float = 1e-5, stats: bool = False, write_sum: bool = True, stream=None):
    """h = x + r, y = RMSNorm(h).  Returns (y, h) or (y, h, rstd)."""
    y, h, _, rstd = _norm(OP_ADD_RMSNORM, x, r, w, None, eps, stats, None, write_sum, stream)
    return (y, h, rstd) if stats else (y, h)


def _norm_bwd(op, dy, x, p0, mean, rstd, param_grads, out, stream):
    import torch
    dt = _dtype_code(x)
    if dy.dtype != x.dtype or dy.shape != x.shape:
        raise ValueError("dy must have x's shape and dtype")
    d = x.shape[-1]
    if out is not None:
        _rows_of(out, "out")
    dy, x = _input_rows(dy), _input_rows(x)
    rows, ldx = _rows_of(x, "x")
    lddy = _rows_of(dy, "dy")[1]
    ctx, handle = _on_stream(stream, x.device)
    with ctx:
        dx = torch.empty(x.shape, device=x.device, dtype=x.dtype) if out is None else out
        if dx.dtype != x.dtype or dx.shape != x.shape:
            raise ValueError("out must have x's shape and dtype")
        lddx = _rows_of(dx, "out")[1]
        ln = op == OP_LAYERNORM
        for t, name in ((mean, "mean"), (rstd, "rstd")):
            if t is None:
                continue
            if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != rows:
                raise ValueError(f"{name} must be a contiguous float32 tensor of one value per row")
        dp0 = torch.empty(d, device=x.device, dtype=torch.float32) if param_grads else None
        dp1 = torch.empty(d, device=x.device, dtype=torch.float32) if (param_grads and ln) else None
        p = bwd_problem(op, rows, d, dy, x, dx, _params(p0, "gamma" if ln else "w", d), mean, rstd, dp0, dp1,
                        dtype=dt, lddy=lddy, ldx=ldx, lddx=lddx)
        nbytes = mi_norm_bwd_workspace_size(p)
        ws = torch.empty(max(nbytes, 1), device=x.device, dtype=torch.uint8) if nbytes > 0 else None
        p.workspace, p.workspace_bytes = (ws.data_ptr() if ws is not None else None), max(nbytes, 0)
        mi_norm_bwd(p, handle)
    return dx, dp0, dp1


def layernorm_bwd(dy, x, gamma, mean, rstd, param_grads: bool = True, out=None, stream=None):
    """LayerNorm backward from the forward's mean/rstd: returns (dx, dgamma,
    dbeta), the parameter gradients None without ``param_grads``.  ``out``
    may be dy or x (in place).  The workspace is a torch allocation."""
    return _norm_bwd(OP_LAYERNORM, dy, x, gamma, mean, rstd, param_grads, out, stream)


def rmsnorm_bwd(dy, x, w, rstd, param_grads: bool = True, out=None, stream=None):
    """RMSNorm backward from the forward's rstd: returns (dx, dw)."""
    dx, dw, _ = _norm_bwd(OP_RMSNORM, dy, x, w, None, rstd, param_grads, out, stream)
    return dx, dw


def rmsnorm(x, w, eps: float = 1e-5, stats: bool = False, out=None, stream=None):
    """RMSNorm over the last dimension; returns y, or (y, rstd) with ``stats``."""
    y, _, _, rstd = _norm(OP_RMSNORM, x, None, w, None, eps, stats, out, False, stream)
    return (y, rstd) if stats else y
