"""GPU parity for 16-bit row storage (binary16, bfloat16) and strided rows,
through the general C call (mi_norm_fwd) against the float64 oracle.

Acceptance: a 16-bit y is within the float32 bound 1e-5 + 1e-4 |ref| of
"RMSNorm on an RTX 5070" (section "Correctness before timing") plus half a
16-bit ulp, measured from the oracle's float64 value before its rounding
(oracle.tolerance_ok16); mean and rstd (float32) within the float32 bound; h
bit for bit.  Row tensors live in buffers whose guard regions AND inter-row
gaps hold a sentinel that must survive.  Every case prints its name first.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import row_wise_normalization_layernorm_amd as mn
from row_wise_normalization_layernorm_amd import workloads as wl

pytestmark = pytest.mark.gpu

GUARD = 512
# sentinels: float32 -31415.5; binary16 65504 (its largest finite value);
# bfloat16 ~3.39e38 (its largest finite value)
SENT = {mn.MI_NORM_F32: np.float32(-31415.5).view(np.uint32), mn.MI_NORM_F16: np.uint16(0x7BFF),
        mn.MI_NORM_BF16: np.uint16(0x7F7F)}
FMT = {mn.MI_NORM_F16: oracle.FMT_F16, mn.MI_NORM_BF16: oracle.FMT_BF16}
OPS = {"layernorm": mn.OP_LAYERNORM, "rmsnorm": mn.OP_RMSNORM, "add_layernorm": mn.OP_ADD_LAYERNORM,
       "add_rmsnorm": mn.OP_ADD_RMSNORM}


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    mn.lib()
    return torch, torch.device("cuda:0")


def say(msg: str) -> None:
    print(msg, flush=True)


class GuardedRows:
    """[rows, d] elements of one storage type at row stride ld, placed `off`
    elements into a device buffer; everything else in the buffer (guards on
    both sides, the ld - d gap after every row) holds the sentinel."""

    def __init__(self, torch, dev, dt: int, rows: int, d: int, ld: int, off: int = 0, init=None):
        self.torch, self.dt, self.rows, self.d, self.ld = torch, dt, rows, d, ld
        self.np_bits = np.uint32 if dt == mn.MI_NORM_F32 else np.uint16
        self.es = 4 if dt == mn.MI_NORM_F32 else 2
        self.base = GUARD + off
        span = (rows - 1) * ld + d if rows else 0
        self.total = self.base + span + GUARD
        host = np.full(self.total, SENT[dt], self.np_bits)
        self.idx = (self.base + np.arange(rows)[:, None] * ld + np.arange(d)[None, :]).reshape(-1)
        if init is not None:
            host[self.idx] = np.ascontiguousarray(init).view(self.np_bits).reshape(-1)
        tdt = torch.int32 if self.es == 4 else torch.int16
        self.buf = torch.from_numpy(host.view(np.int32 if self.es == 4 else np.int16)).to(dev)
        assert self.buf.dtype == tdt

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr() + self.base * self.es

    def bits(self) -> np.ndarray:
        return self.buf.cpu().numpy().view(self.np_bits)

    def rows_host(self) -> np.ndarray:
        """The [rows, d] data (float32 values, or 16-bit patterns)."""
        b = self.bits()[self.idx].reshape(self.rows, self.d)
        return b.view(np.float32) if self.es == 4 else b

    def intact(self) -> bool:
        b = self.bits()
        mask = np.ones(self.total, bool)
        mask[self.idx] = False
        return bool(np.all(b[mask] == SENT[self.dt]))


class GuardedVec:
    """A float32 [n] vector at a float offset with sentinel guards."""

    def __init__(self, torch, dev, n: int, off: int = 0, init=None):
        self.n, self.base = n, GUARD + off
        host = np.full(self.base + n + GUARD, np.float32(-31415.5), np.float32)
        if init is not None:
            host[self.base:self.base + n] = init
        self.buf = torch.from_numpy(host).to(dev)

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr() + 4 * self.base

    def host(self) -> np.ndarray:
        return self.buf.cpu().numpy()[self.base:self.base + self.n]

    def intact(self) -> bool:
        b = self.buf.cpu().numpy()
        return bool(np.all(b[:self.base] == np.float32(-31415.5)) and
                    np.all(b[self.base + self.n:] == np.float32(-31415.5)))


def inputs(op: str, dt: int, rows: int, d: int, pattern: str, seed):
    """x (and r) in the storage type (float32 values or 16-bit patterns), the
    float32 parameters."""
    x = wl.make_x(rows, d, pattern, seed)
    r = wl.make_x(rows, d, "normal", [9] + list(seed)) if op.startswith("add_") else None
    if dt != mn.MI_NORM_F32:
        x = wl.quantize16(x, FMT[dt])
        r = None if r is None else wl.quantize16(r, FMT[dt])
    params = wl.make_affine(d, [9, d]) if op.endswith("layernorm") else (wl.make_weight(d, [9, d]),)
    return x, r, params


def oracle_ref(op: str, dt: int, x, r, params, eps):
    """dict of expected outputs: y (float32 values or 16-bit float64 y64), h, mean, rstd."""
    if dt == mn.MI_NORM_F32:
        if op == "layernorm":
            y, m, s, _, _ = oracle.layernorm(x, *params, eps)
            return dict(y=y, mean=m, rstd=s)
        if op == "rmsnorm":
            y, s, _ = oracle.rmsnorm(x, *params, eps)
            return dict(y=y, rstd=s)
        if op == "add_layernorm":
            y, h, m, s = oracle.add_layernorm(x, r, *params, eps)
            return dict(y=y, h=h, mean=m, rstd=s)
        y, h, s = oracle.add_rmsnorm(x, r, *params, eps)
        return dict(y=y, h=h, rstd=s)
    f = FMT[dt]
    if op == "layernorm":
        _, y64, m, s = oracle.layernorm16(x, f, *params, eps)
        return dict(y64=y64, mean=m, rstd=s)
    if op == "rmsnorm":
        _, y64, s = oracle.rmsnorm16(x, f, *params, eps)
        return dict(y64=y64, rstd=s)
    if op == "add_layernorm":
        _, y64, h, m, s = oracle.add_layernorm16(x, r, f, *params, eps)
        return dict(y64=y64, h=h, mean=m, rstd=s)
    _, y64, h, s = oracle.add_rmsnorm16(x, r, f, *params, eps)
    return dict(y64=y64, h=h, rstd=s)


def run_case(torch, dev, op: str, dt: int, x, r, params, *, ld=None, off=None, po: int = 0,
             y_mode=None, h_mode="new", variant=None, stats=True, eps=wl.EPS) -> float:
    """One call of mi_norm_fwd (or mi_norm_fwd_variant) on guarded strided
    buffers, checked against the oracle.  ld / off: per-tensor row stride and
    element offset dicts over 'x', 'r', 'y', 'h'.  y_mode / h_mode as in
    test_parity.run_case ('x' or 'r' writes over that input; h 'none' skips)."""
    rows, d = x.shape
    add = op.startswith("add_")
    ln = op.endswith("layernorm")
    ld = {k: d for k in "xryh"} | (ld or {})
    off = {k: 0 for k in "xryh"} | (off or {})
    X = GuardedRows(torch, dev, dt, rows, d, ld["x"], off["x"], x)
    R = GuardedRows(torch, dev, dt, rows, d, ld["r"], off["r"], r) if add else None
    ins = {"x": (X, ld["x"]), "r": (R, ld["r"])}
    Y, ldy = ins[y_mode] if y_mode else (GuardedRows(torch, dev, dt, rows, d, ld["y"], off["y"]), ld["y"])
    H, ldh = None, 0
    if add and h_mode != "none":
        H, ldh = ins[h_mode] if h_mode in ("x", "r") else (GuardedRows(torch, dev, dt, rows, d, ld["h"], off["h"]),
                                                        ld["h"])
    P = [GuardedVec(torch, dev, d, po, p) for p in params]
    M = GuardedVec(torch, dev, rows) if (stats and ln) else None
    S = GuardedVec(torch, dev, rows) if stats else None
    prob = mn.problem(OPS[op], rows, d, X.ptr, Y.ptr, P[0].ptr, P[1].ptr if ln else None,
                      r=R.ptr if add else None, h=H.ptr if H else None, dtype=dt, ldx=ld["x"],
                      ldr=ld["r"] if add else 0, ldy=ldy, ldh=ldh, eps=eps,
                      mean=M.ptr if M else None, rstd=S.ptr if S else None)
    stream = torch.cuda.current_stream().cuda_stream
    if variant is None:
        mn.mi_norm_fwd(prob, stream)
    else:
        mn.mi_norm_fwd_variant(variant, prob, stream)
    torch.cuda.synchronize()
    ref = oracle_ref(op, dt, x, r, params, eps)
    worst = 0.0
    got_y = Y.rows_host()
    if dt == mn.MI_NORM_F32:
        ok, err, ratio = oracle.tolerance_ok(got_y, ref["y"])
    else:
        ok, err, ratio = oracle.tolerance_ok16(got_y, ref["y64"], FMT[dt])
    assert ok, f"y: max abs err {err:.3e}, err/bound {ratio:.3f}"
    worst = max(worst, err)
    for buf, key in ((M, "mean"), (S, "rstd")):
        if buf is None:
            continue
        ok, err, ratio = oracle.tolerance_ok(buf.host(), ref[key])
        assert ok, f"{key}: max abs err {err:.3e}, err/bound {ratio:.3f}"
        assert buf.intact(), f"{key}: write outside its range"
    if H is not None:
        got_h = H.rows_host()
        assert np.array_equal(got_h.view(np.uint32 if dt == mn.MI_NORM_F32 else np.uint16),
                              ref["h"].view(np.uint32 if dt == mn.MI_NORM_F32 else np.uint16)), "h != x + r"
    for g, what in ((X, "x"), (R, "r"), (Y, "y"), (H, "h")):
        if g is not None:
            assert g.intact(), f"{what}: write outside its rows (guards or row gaps)"
    for p in P:
        assert p.intact()
    if y_mode != "x" and h_mode != "x":
        assert np.array_equal(X.rows_host().view(X.np_bits), np.asarray(x).view(X.np_bits)), "x was modified"
    if add and y_mode != "r" and h_mode != "r":
        assert np.array_equal(R.rows_host().view(R.np_bits), np.asarray(r).view(R.np_bits)), "r was modified"
    return worst


DT16 = [pytest.param(mn.MI_NORM_F16, id="f16"), pytest.param(mn.MI_NORM_BF16, id="bf16")]


# --- 16-bit storage over the pages' shapes and patterns ------------------------

@pytest.mark.parametrize("dt", DT16)
@pytest.mark.parametrize("op", list(OPS))
def test_storage16_shapes(torch_dev, dt, op):
    torch, dev = torch_dev
    shapes = [(512, 128, p) for p in ("normal", "zero", "tiny", "alternating")]
    shapes += [(64, d, p) for d in (1, 31, 33, 127) for p in ("normal", "alternating")]
    shapes += [(4096, 768, "normal"), (8192, 768, "offset"), (1024, 2048, "offset"), (2048, 4096, "normal"),
               (256, 8193, "normal"), (64, 2049, "offset")]
    for rows, d, pat in shapes:
        say(f"storage16 {op} dt={dt} [{rows}x{d}] {pat}")
        x, r, params = inputs(op, dt, rows, d, pat, [10, rows, d])
        run_case(torch, dev, op, dt, x, r, params)


@pytest.mark.parametrize("dt", DT16)
def test_storage16_wide_rows(torch_dev, dt):
    """Widths past the held variants (streamed rows) and near the caps."""
    torch, dev = torch_dev
    for op, rows, d in (("layernorm", 5, 40000), ("add_rmsnorm", 3, 65536), ("add_layernorm", 4, 32768),
                        ("rmsnorm", 7, 40001)):
        say(f"storage16 wide {op} dt={dt} [{rows}x{d}]")
        x, r, params = inputs(op, dt, rows, d, "offset", [11, rows, d])
        run_case(torch, dev, op, dt, x, r, params)


@pytest.mark.parametrize("dt", DT16)
def test_storage16_full_size(torch_dev, dt):
    """[32768, 8192] in a 16-bit type through the dispatcher; sampled rows
    checked against the oracle (the whole output would take minutes on the
    CPU), every row's statistics finite and every guard intact."""
    torch, dev = torch_dev
    rows, d = 32768, 8192
    say(f"storage16 full size dt={dt} [{rows}x{d}]")
    x32 = torch.randn(rows, d, device=dev, generator=torch.Generator(device=dev).manual_seed(12))
    x = x32.to(torch.float16 if dt == mn.MI_NORM_F16 else torch.bfloat16)
    g, b = (torch.from_numpy(a).to(dev) for a in wl.make_affine(d, [12, d]))
    y, mean, rstd = mn.layernorm(x, g, b, wl.EPS, stats=True)
    torch.cuda.synchronize()
    sample = np.unique(np.random.default_rng(12).integers(0, rows, 256))
    xs = x[torch.from_numpy(sample).to(dev)].cpu().view(torch.int16).numpy().view(np.uint16)
    _, y64, m, s = oracle.layernorm16(xs, FMT[dt], g.cpu().numpy(), b.cpu().numpy(), wl.EPS)
    ys = y[torch.from_numpy(sample).to(dev)].cpu().view(torch.int16).numpy().view(np.uint16)
    ok, err, ratio = oracle.tolerance_ok16(ys, y64, FMT[dt])
    assert ok, f"y: max abs err {err:.3e}, err/bound {ratio:.3f}"
    assert oracle.tolerance_ok(mean.cpu().numpy()[sample], m)[0]
    assert oracle.tolerance_ok(rstd.cpu().numpy()[sample], s)[0]
    assert bool(torch.isfinite(rstd).all()) and bool(torch.isfinite(mean).all())


# --- every compiled 16-bit variant, forced, on strided rows -------------------

def _variant_widths(v):
    if v["looped"]:
        return [v["vec"] * 1237, 40000] if v["vec"] > 1 else [4947, 40001]
    cap = v["max_d"]
    if v["peel"]:
        return sorted(w for w in {cap, cap - 1 - 4 * 64, max(128, cap // 3 - 1), 128} if w >= 128)
    step = v["vec"]
    return sorted(w for w in {cap, cap - step * max(1, cap // (7 * step)), step} if w >= 1)


def _variant_layouts(v, d):
    """Row strides and offsets that the variant accepts, with gaps between rows."""
    if v["needs_aligned"]:
        return [dict(ld={k: d + 8 for k in "xryh"}, off={k: 0 for k in "xryh"}, po=0)]
    if v["peel"]:
        # one phase within 16 bytes on every row (equal offsets, strides equal
        # mod 8 elements: the body starts on a 16-byte boundary), and one phase
        # within a cache line (strides equal mod 64 elements: the body starts
        # on a line, after a head of up to 31 or 63 elements)
        return [dict(ld={"x": d + 5, "r": d + 13, "y": d + 21, "h": d + 5}, off={k: 1 for k in "xryh"}, po=2),
                dict(ld={"x": d + 5, "r": d + 69, "y": d + 133, "h": d + 5}, off={k: 3 for k in "xryh"}, po=1)]
    return [dict(ld={"x": d + 3, "r": d + 2, "y": d + 1, "h": d + 7}, off={"x": 1, "r": 2, "y": 3, "h": 0}, po=3)]


OPNAME = {v: k for k, v in OPS.items()}


@pytest.mark.parametrize("dt", [pytest.param(mn.MI_NORM_F32, id="f32")] + DT16)
def test_every_variant_strided(torch_dev, dt):
    torch, dev = torch_dev
    n = 0
    for vid in range(mn.mi_norm_variant_count()):
        v = mn.mi_norm_variant_get_info(vid)
        if v["dtype"] != dt or v["op"] not in OPNAME:
            continue                     # backward variants: test_parity_bwd.py
        name = mn.mi_norm_variant_name(vid)
        op = OPNAME[v["op"]]
        for d in _variant_widths(v):
            rows = min(3 * v["rows_per_block"] + 1, max(2, 300000 // d))
            for lay in _variant_layouts(v, d):
                say(f"variant {vid} {name} rows={rows} d={d} {lay}")
                x, r, params = inputs(op, dt, rows, d, "offset", [13, vid, d])
                run_case(torch, dev, op, dt, x, r, params, variant=vid, **lay)
                n += 1
    assert n > 0


# --- strided rows through the dispatcher --------------------------------------

@pytest.mark.parametrize("dt", [pytest.param(mn.MI_NORM_F32, id="f32")] + DT16)
@pytest.mark.parametrize("op", list(OPS))
@pytest.mark.parametrize("d,pad", [(768, 256), (768, 3), (2049, 7), (127, 1), (8192, 64), (40000, 8)])
def test_strided_rows(torch_dev, dt, op, d, pad):
    torch, dev = torch_dev
    rows = 37 if d < 10000 else 5
    say(f"strided {op} dt={dt} d={d} pad={pad}")
    x, r, params = inputs(op, dt, rows, d, "offset", [14, d, pad])
    run_case(torch, dev, op, dt, x, r, params, ld={"x": d + pad, "r": d + 2 * pad, "y": d + pad, "h": d})


@pytest.mark.parametrize("dt", [pytest.param(mn.MI_NORM_F32, id="f32")] + DT16)
def test_interleaved_inputs_and_outputs(torch_dev, dt):
    """x and r interleaved in one [rows, 2d] buffer, and y, h interleaved in
    another: no shared element, so the library accepts both."""
    torch, dev = torch_dev
    rows, d = 300, 1024
    say(f"interleaved dt={dt}")
    x, r, params = inputs("add_layernorm", dt, rows, d, "normal", [15])
    es = 4 if dt == mn.MI_NORM_F32 else 2
    XR = GuardedRows(torch, dev, dt, rows, 2 * d, 2 * d, 0,
                     np.concatenate([np.asarray(x), np.asarray(r)], axis=1))
    YH = GuardedRows(torch, dev, dt, rows, 2 * d, 2 * d, 0)
    P = [GuardedVec(torch, dev, d, 0, p) for p in params]
    prob = mn.problem(mn.OP_ADD_LAYERNORM, rows, d, XR.ptr, YH.ptr, P[0].ptr, P[1].ptr, r=XR.ptr + es * d,
                      h=YH.ptr + es * d, dtype=dt, ldx=2 * d, ldr=2 * d, ldy=2 * d, ldh=2 * d, eps=wl.EPS)
    mn.mi_norm_fwd(prob)
    torch.cuda.synchronize()
    ref = oracle_ref("add_layernorm", dt, x, r, params, wl.EPS)
    out = YH.rows_host()
    y, h = out[:, :d], out[:, d:]
    if dt == mn.MI_NORM_F32:
        assert oracle.tolerance_ok(y, ref["y"])[0]
        assert np.array_equal(h.view(np.uint32), ref["h"].view(np.uint32))
    else:
        assert oracle.tolerance_ok16(np.ascontiguousarray(y), ref["y64"], FMT[dt])[0]
        assert np.array_equal(h, ref["h"])
    assert XR.intact() and YH.intact()


@pytest.mark.parametrize("dt", DT16)
@pytest.mark.parametrize("y_mode,h_mode", [("x", "new"), (None, "x"), ("r", "x"), ("x", "r"), (None, "none")])
def test_storage16_in_place(torch_dev, dt, y_mode, h_mode):
    torch, dev = torch_dev
    for op in ("add_layernorm", "add_rmsnorm"):
        for d in (768, 2049, 40000):
            rows = 33 if d < 10000 else 3
            say(f"storage16 in place {op} dt={dt} d={d} y={y_mode} h={h_mode}")
            x, r, params = inputs(op, dt, rows, d, "offset", [16, d])
            run_case(torch, dev, op, dt, x, r, params, y_mode=y_mode, h_mode=h_mode,
                     ld={"x": d + 4, "r": d + 4, "y": d + 4, "h": d + 4})


def test_binding_takes_torch_16bit_and_strided_views(torch_dev):
    """The torch conveniences pass dtype and row stride straight through."""
    torch, dev = torch_dev
    base = torch.randn(64, 1000, device=dev).to(torch.bfloat16)
    x = base[:, 100:868]                     # [64, 768] rows at stride 1000
    g, b = (torch.from_numpy(a).to(dev) for a in wl.make_affine(768, [17]))
    say("binding bf16 strided view")
    y, mean, rstd = mn.layernorm(x, g, b, wl.EPS, stats=True)
    torch.cuda.synchronize()
    xs = x.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    _, y64, m, s = oracle.layernorm16(xs, oracle.FMT_BF16, g.cpu().numpy(), b.cpu().numpy(), wl.EPS)
    assert oracle.tolerance_ok16(y.cpu().view(torch.int16).numpy().view(np.uint16), y64, oracle.FMT_BF16)[0]
    assert oracle.tolerance_ok(mean.cpu().numpy(), m)[0]
    with pytest.raises(ValueError):
        mn.layernorm(x, g.to(torch.bfloat16), b, wl.EPS)    # parameters are float32
