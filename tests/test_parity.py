"""GPU parity: the HIP library (through its C ABI) against the float64 oracle.

Acceptance is elementwise |gpu - ref| <= 1e-5 + 1e-4 |ref| on y, mean and rstd
with no NaN/Inf, the bound of "RMSNorm on an RTX 5070" (section "Correctness
before timing").  Outputs sit between guard regions filled with a sentinel
that must survive, as on that page.  Every case prints its name first.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import row_wise_normalization_layernorm_amd as mn
from row_wise_normalization_layernorm_amd import workloads as wl

pytestmark = pytest.mark.gpu

GUARD = 1024          # floats of guard on each side of every output
SENTINEL = -31415.5   # survives only if nothing writes outside its range


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    mn.lib()
    return torch, torch.device("cuda:0")


def say(msg: str) -> None:
    print(msg, flush=True)


class Guarded:
    """A device float32 buffer of n elements at a chosen float offset, with
    sentinel-filled guard regions around it."""

    def __init__(self, torch, dev, n: int, offset: int = 0, init: np.ndarray | None = None):
        self.torch, self.n, self.off = torch, n, GUARD + offset
        self.buf = torch.full((2 * GUARD + n + 4,), SENTINEL, dtype=torch.float32, device=dev)
        self.view = self.buf[self.off:self.off + n]
        if init is not None:
            self.view.copy_(torch.from_numpy(np.ascontiguousarray(init).reshape(-1)))

    @property
    def ptr(self) -> int:
        return self.view.data_ptr()

    def host(self) -> np.ndarray:
        return self.view.cpu().numpy()

    def guards_intact(self) -> bool:
        b = self.buf.cpu().numpy()
        return bool(np.all(b[:self.off] == SENTINEL) and np.all(b[self.off + self.n:] == SENTINEL))


def check(got, ref, what: str):
    ok, err, ratio = oracle.tolerance_ok(got, ref)
    assert ok, f"{what}: max abs err {err:.3e}, worst err/bound {ratio:.3f}"
    return err


def run_case(torch, dev, op, x, params, eps=wl.EPS, stats=True, variant=None, xo=0, yo=None,
             po=0, inplace=False, r=None, h_mode="new", y_mode=None):
    """Run one case through the C ABI with guarded buffers; compare with the oracle.

    Fused ops take the residual r; h_mode is "new" (a buffer of its own),
    "none" (not written), "x" or "r" (written over that input); y_mode "x" or
    "r" writes y over that input (``inplace`` is y_mode "x")."""
    rows, d = x.shape
    yo = xo if yo is None else yo
    add = op.startswith("add_")
    ln = op.endswith("layernorm")
    y_mode = "x" if inplace else y_mode
    X = Guarded(torch, dev, rows * d, xo, x)
    Rr = Guarded(torch, dev, rows * d, xo, r) if add else None
    bufs = {"x": X, "r": Rr}
    Y = bufs[y_mode] if y_mode else Guarded(torch, dev, rows * d, yo)
    Hh = None
    if add and h_mode != "none":
        Hh = bufs[h_mode] if h_mode in ("x", "r") else Guarded(torch, dev, rows * d, yo)
    P = [Guarded(torch, dev, d, po, p) for p in params]
    M = Guarded(torch, dev, rows) if (stats and ln) else None
    R = Guarded(torch, dev, rows) if stats else None
    L = mn.lib()
    st = torch.cuda.current_stream().cuda_stream
    mp, rp = (M.ptr if M else None), (R.ptr if R else None)
    hp = Hh.ptr if Hh else None
    if op == "layernorm":
        s = (L.mi_layernorm_fwd(X.ptr, P[0].ptr, P[1].ptr, Y.ptr, rows, d, eps, mp, rp, st) if variant is None
             else L.mi_layernorm_fwd_variant(variant, X.ptr, P[0].ptr, P[1].ptr, Y.ptr, rows, d, eps, mp, rp, st))
        ref = oracle.layernorm(x, *params, eps)
        refs = [(Y, ref[0].reshape(-1), "y"), (M, ref[1], "mean"), (R, ref[2], "rstd")]
        ref_h = None
    elif op == "rmsnorm":
        s = (L.mi_rmsnorm_fwd(X.ptr, P[0].ptr, Y.ptr, rows, d, eps, rp, st) if variant is None
             else L.mi_rmsnorm_fwd_variant(variant, X.ptr, P[0].ptr, Y.ptr, rows, d, eps, rp, st))
        ref = oracle.rmsnorm(x, *params, eps)
        refs = [(Y, ref[0].reshape(-1), "y"), (R, ref[1], "rstd")]
        ref_h = None
    elif op == "add_layernorm":
        s = (L.mi_add_layernorm_fwd(X.ptr, Rr.ptr, P[0].ptr, P[1].ptr, Y.ptr, hp, rows, d, eps, mp, rp, st)
             if variant is None else
             L.mi_add_layernorm_fwd_variant(variant, X.ptr, Rr.ptr, P[0].ptr, P[1].ptr, Y.ptr, hp, rows, d,
                                            eps, mp, rp, st))
        ref = oracle.add_layernorm(x, r, *params, eps)
        refs = [(Y, ref[0].reshape(-1), "y"), (M, ref[2], "mean"), (R, ref[3], "rstd")]
        ref_h = ref[1].reshape(-1)
    else:
        s = (L.mi_add_rmsnorm_fwd(X.ptr, Rr.ptr, P[0].ptr, Y.ptr, hp, rows, d, eps, rp, st)
             if variant is None else
             L.mi_add_rmsnorm_fwd_variant(variant, X.ptr, Rr.ptr, P[0].ptr, Y.ptr, hp, rows, d, eps, rp, st))
        ref = oracle.add_rmsnorm(x, r, *params, eps)
        refs = [(Y, ref[0].reshape(-1), "y"), (R, ref[2], "rstd")]
        ref_h = ref[1].reshape(-1)
    assert s == mn.MI_NORM_OK, mn.mi_norm_status_string(s)
    torch.cuda.synchronize()
    worst = 0.0
    for buf, want, what in refs:
        if buf is None:
            continue
        worst = max(worst, check(buf.host(), want, what))
        assert buf.guards_intact(), f"{what}: write outside the output range"
    if Hh is not None:
        # the same IEEE float32 addition on both sides: bit for bit
        assert np.array_equal(Hh.host(), ref_h), "h != x + r"
        assert Hh.guards_intact(), "h: write outside the output range"
    for p in P:
        assert p.guards_intact()
    if y_mode != "x" and h_mode != "x":
        assert np.array_equal(X.host(), x.reshape(-1)), "x was modified"
    if add and y_mode != "r" and h_mode != "r":
        assert np.array_equal(Rr.host(), r.reshape(-1)), "r was modified"
    return worst


# --- the workload families ----------------------------------------------------

@pytest.mark.parametrize("name", ["ln_small", "ln_4096x768", "ln_sweep", "rms", "residual"])
def test_workload_family(torch_dev, name):
    torch, dev = torch_dev
    for case in wl.WORKLOADS[name].cases:
        say(f"case {case.name}")
        a = case.arrays()
        err = run_case(torch, dev, case.op, a["x"], a["params"], stats=True, r=a["r"])
        say(f"  max abs err {err:.3e}")


def test_ln_32768x8192_full_size(torch_dev):
    """The bandwidth-saturating shape, every output compared, in the default
    dispatch the benchmark times."""
    torch, dev = torch_dev
    case = wl.WORKLOADS["ln_32768x8192"].cases[0]
    say(f"case {case.name}")
    x, g, b = case.inputs()
    rows, d = x.shape
    xd = torch.from_numpy(x).to(dev)
    yd = torch.empty_like(xd)
    mean = torch.empty(rows, device=dev)
    rstd = torch.empty(rows, device=dev)
    mn.mi_layernorm_fwd(xd, torch.from_numpy(g).to(dev), torch.from_numpy(b).to(dev), yd, rows, d,
                        wl.EPS, mean, rstd)
    torch.cuda.synchronize()
    y = yd.cpu().numpy()
    del yd, xd
    ry, rm, rr, _, _ = oracle.layernorm(x, g, b, wl.EPS)
    for r0 in range(0, rows, 4096):
        check(y[r0:r0 + 4096], ry[r0:r0 + 4096], f"y rows {r0}..")
    check(mean.cpu().numpy(), rm, "mean")
    check(rstd.cpu().numpy(), rr, "rstd")


# --- every compiled variant, forced ------------------------------------------

def _variant_widths(v):
    """Widths that fill a variant exactly, leave a ragged last slot, and are small."""
    if v["looped"]:
        return [4 * 1237, 40000] if v["vec"] == 4 else [4947, 40001]
    cap = v["max_d"]
    if v["peel"]:
        # a body that fills the variant with the widest tail, a ragged one,
        # and the narrowest row a peeled variant takes (128)
        return sorted(w for w in {cap, cap - 4, cap - 1 - 4 * 64, max(128, cap // 3 - 1), 128} if w >= 128)
    step = 4 if v["vec"] == 4 else 1
    widths = {cap, cap - step * max(1, cap // (7 * step)), step}
    return sorted(w for w in widths if w >= 1)


def _variant_layout(v):
    if v["needs_aligned"]:
        return dict(xo=0, yo=0, po=0)
    if v["peel"]:
        return dict(xo=1, yo=1, po=2)   # x and y share their phase (within a cache line: a head of 31)
    return dict(xo=1, yo=2, po=3)       # nothing aligned


OPNAME = {mn.OP_LAYERNORM: "layernorm", mn.OP_RMSNORM: "rmsnorm",
          mn.OP_ADD_LAYERNORM: "add_layernorm", mn.OP_ADD_RMSNORM: "add_rmsnorm"}


def test_every_variant(torch_dev):
    """Every float32 variant through the named calls on contiguous rows (the
    16-bit variants, and strided rows, are in test_parity_storage.py)."""
    torch, dev = torch_dev
    n = mn.mi_norm_variant_count()
    for vid in range(n):
        v = mn.mi_norm_variant_get_info(vid)
        if v["dtype"] != mn.MI_NORM_F32 or v["op"] not in OPNAME:
            continue                     # 16-bit and backward variants: their own tests
        name = mn.mi_norm_variant_name(vid)
        op = OPNAME[v["op"]]
        lay = _variant_layout(v)
        for d in _variant_widths(v):
            rows = min(3 * v["rows_per_block"] + 1, max(2, 600000 // d))
            say(f"variant {vid} {name} rows={rows} d={d} {lay}")
            x = wl.make_x(rows, d, "offset", [7, vid, d])
            r = wl.make_x(rows, d, "normal", [8, vid, d]) if op.startswith("add_") else None
            params = wl.make_affine(d, [7, d]) if op.endswith("layernorm") else (wl.make_weight(d, [7, d]),)
            run_case(torch, dev, op, x, params, variant=vid, r=r, **lay)


@pytest.mark.parametrize("pattern", ["normal", "alternating", "tiny", "offset"])
@pytest.mark.parametrize("op", ["layernorm", "add_layernorm"])
def test_streamed_rows_patterns(torch_dev, op, pattern):
    """Rows past the held variants (the streamed kernel, whose LayerNorm
    statistics merge per-chunk centered sums) on the pages' four patterns."""
    torch, dev = torch_dev
    for rows, d in ((5, 40000), (3, 65536), (2, 98307)):
        say(f"streamed {op} [{rows}x{d}] {pattern}")
        x = wl.make_x(rows, d, pattern, [61, rows, d])
        r = wl.make_x(rows, d, "normal", [62, rows, d]) if op.startswith("add_") else None
        run_case(torch, dev, op, x, wl.make_affine(d, [61, d]), r=r, xo=0 if d % 4 == 0 else 1)


# --- layouts, aliasing, ordering ---------------------------------------------

@pytest.mark.parametrize("op", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("d,xo,yo,po", [(768, 0, 0, 0), (768, 1, 1, 0), (768, 1, 2, 0),
                                        (768, 0, 0, 1), (8193, 0, 0, 0), (8193, 3, 3, 1),
                                        (4096, 2, 0, 0), (33, 1, 3, 2), (1, 0, 0, 0)])
def test_layouts_dispatch(torch_dev, op, d, xo, yo, po):
    torch, dev = torch_dev
    rows = 37
    say(f"layout {op} d={d} xo={xo} yo={yo} po={po}")
    x = wl.make_x(rows, d, "offset", [8, d, xo, yo])
    params = wl.make_affine(d, [8, d]) if op == "layernorm" else (wl.make_weight(d, [8, d]),)
    run_case(torch, dev, op, x, params, xo=xo, yo=yo, po=po)


@pytest.mark.parametrize("op", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("d,xo", [(768, 0), (2049, 1), (127, 3), (16384, 0)])
def test_in_place(torch_dev, op, d, xo):
    torch, dev = torch_dev
    say(f"in place {op} d={d} xo={xo}")
    x = wl.make_x(45, d, "normal", [9, d])
    params = wl.make_affine(d, [9, d]) if op == "layernorm" else (wl.make_weight(d, [9, d]),)
    run_case(torch, dev, op, x, params, xo=xo, inplace=True)


@pytest.mark.parametrize("op", ["add_layernorm", "add_rmsnorm"])
@pytest.mark.parametrize("d,xo", [(768, 0), (2049, 1), (127, 3), (40000, 0)])
@pytest.mark.parametrize("y_mode,h_mode", [(None, "new"), (None, "none"), ("x", "new"), ("r", "new"),
                                           (None, "x"), (None, "r"), ("x", "r"), ("r", "x")])
def test_residual_aliasing(torch_dev, op, d, xo, y_mode, h_mode):
    """y and h written over the inputs in every allowed combination."""
    torch, dev = torch_dev
    rows = 37 if d < 10000 else 5
    say(f"residual aliasing {op} d={d} xo={xo} y={y_mode} h={h_mode}")
    x = wl.make_x(rows, d, "offset", [12, d])
    r = wl.make_x(rows, d, "normal", [13, d])
    params = wl.make_affine(d, [12, d]) if op == "add_layernorm" else (wl.make_weight(d, [12, d]),)
    run_case(torch, dev, op, x, params, xo=xo, r=r, y_mode=y_mode, h_mode=h_mode)


def test_without_stats_and_eps_zero(torch_dev):
    torch, dev = torch_dev
    say("no stats, eps = 0")
    x = wl.make_x(64, 768, "normal", [10])
    g, b = wl.make_affine(768, [10])
    run_case(torch, dev, "layernorm", x, (g, b), eps=0.0, stats=False)
    run_case(torch, dev, "rmsnorm", x, (g,), eps=0.0, stats=False)


def test_stream_ordering(torch_dev):
    """Work enqueued on a side stream runs after the torch op that produced x."""
    torch, dev = torch_dev
    say("stream ordering")
    rows, d = 2048, 1024
    x = wl.make_x(rows, d, "normal", [11])
    g, b = wl.make_affine(d, [11])
    xs = torch.from_numpy(x).to(dev)
    gd, bd = torch.from_numpy(g).to(dev), torch.from_numpy(b).to(dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        xd = torch.empty_like(xs)
        xd.copy_(xs * 2.0)      # produced on s, consumed on s
        yd = torch.empty_like(xd)
        mn.mi_layernorm_fwd(xd, gd, bd, yd, rows, d, wl.EPS, stream=s)
    torch.cuda.synchronize()
    ref = oracle.layernorm((x.astype(np.float64) * 2).astype(np.float32), g, b, wl.EPS)[0]
    check(yd.cpu().numpy(), ref, "y on a side stream")


def test_rows_zero_and_errors_on_device(torch_dev):
    torch, dev = torch_dev
    say("rows = 0, bad args with device pointers")
    x = torch.zeros(4, 8, device=dev)
    g = torch.ones(8, device=dev)
    mn.mi_layernorm_fwd(x, g, g, x, 0, 8)
    with pytest.raises(mn.MiNormError):
        mn.mi_layernorm_fwd(x, g, g, x, 4, 8, eps=-1.0)
    assert torch.all(x == 0)


def test_copy_calibration_kernel(torch_dev):
    """Every size band of the copy's shape table (the bytes moved: up to 16,
    48, 160 and 768 MiB, and beyond), a ragged last workgroup, a length not
    a multiple of four and a misaligned start; nothing past the end written."""
    torch, dev = torch_dev
    for n, off in ((1 << 20, 0), (1000003, 0), (4096, 1), ((4 << 20) + 36, 0), ((12 << 20) + 4, 0),
                   ((48 << 20) + 1028, 0), ((128 << 20) + 8, 0)):
        say(f"copy kernel n={n} off={off}")
        src = torch.randn(n + 64, device=dev)[off:off + n]
        dbuf = torch.full((n + 64,), -7.0, device=dev)
        dst = dbuf[off:off + n]
        mn.mi_copy_f32(src, dst, n)
        torch.cuda.synchronize()
        assert torch.equal(src, dst)
        assert bool((dbuf[off + n:] == -7.0).all()) and bool((dbuf[:off] == -7.0).all())
        del src, dbuf, dst
