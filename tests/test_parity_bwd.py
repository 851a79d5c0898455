"""GPU parity for the LayerNorm / RMSNorm backward (mi_norm_bwd) against the
float64 oracle (oracle.layernorm_bwd / rmsnorm_bwd and their 16-bit forms).

Both sides get the same inputs: dy, x, the parameters, and the per-row
statistics the oracle's forward returns (float32).  Acceptance: dx within
1e-5 + 1e-4 |ref| + 16 u * rstd * (|g| + mean|g| + |xhat| mean|g xhat|) of the
float64 derivative (16-bit dx: plus half a 16-bit ulp; oracle.dx_tolerance_ok);
the parameter gradients, which are float32 sums over rows, within the float32
bound plus 6 u sum|terms| (oracle.colsum_tolerance_ok).  Both bounds follow
from the library's arithmetic contract (terms in float32, sums in float64
but for groups of eight terms of a row, each mean and partial sum rounded
once, at most two levels of partial sums), not from its summation trees.
Every row tensor, vector and the workspace sit between sentinel guards that
must survive; the workspace starts full of NaN.  Every case prints its name.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import row_wise_normalization_layernorm_amd as mn
from row_wise_normalization_layernorm_amd import workloads as wl
from test_parity_storage import FMT, GuardedRows, GuardedVec

pytestmark = pytest.mark.gpu

OPS = {"layernorm": mn.OP_LAYERNORM, "rmsnorm": mn.OP_RMSNORM}
DTS = [pytest.param(mn.MI_NORM_F32, id="f32"), pytest.param(mn.MI_NORM_F16, id="f16"),
       pytest.param(mn.MI_NORM_BF16, id="bf16")]


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    mn.lib()
    return torch, torch.device("cuda:0")


def say(msg: str) -> None:
    print(msg, flush=True)


def bwd_inputs(op: str, dt: int, rows: int, d: int, pattern: str, seed):
    """dy, x (storage type), the float32 parameter and the forward's float32
    statistics (mean, rstd; mean None for RMSNorm) from the oracle's forward."""
    x = wl.make_x(rows, d, pattern, seed)
    dy = wl.make_x(rows, d, "normal", [31] + list(seed))
    p0 = wl.make_affine(d, [31, d])[0] if op == "layernorm" else wl.make_weight(d, [31, d])
    if dt != mn.MI_NORM_F32:
        x, dy = wl.quantize16(x, FMT[dt]), wl.quantize16(dy, FMT[dt])
        xw = oracle.widen16(x, FMT[dt])
    else:
        xw = x
    if op == "layernorm":
        _, mean, rstd, _, _ = oracle.layernorm(xw, p0, np.zeros(d, np.float32), wl.EPS)
    else:
        _, rstd, _ = oracle.rmsnorm(xw, p0, wl.EPS)
        mean = None
    return dy, x, p0, mean, rstd


def bwd_ref(op: str, dt: int, dy, x, p0, mean, rstd) -> dict:
    if dt == mn.MI_NORM_F32:
        return (oracle.layernorm_bwd(dy, x, p0, mean, rstd) if op == "layernorm"
                else oracle.rmsnorm_bwd(dy, x, p0, rstd))
    f = FMT[dt]
    return (oracle.layernorm_bwd16(dy, x, f, p0, mean, rstd) if op == "layernorm"
            else oracle.rmsnorm_bwd16(dy, x, f, p0, rstd))


def run_bwd_case(torch, dev, op: str, dt: int, dy, x, p0, mean, rstd, *, ld=None, off=None, po: int = 0,
                 dx_mode=None, param_grads=True, variant=None, ref=None, expect=None) -> None:
    """One mi_norm_bwd (or forced variant) call on guarded buffers, checked
    against the oracle.  ld / off: per-tensor stride / element offset dicts
    over 'dy', 'x', 'dx'; dx_mode 'dy' or 'x' writes dx over that input;
    expect: the name the dispatcher must choose for this problem."""
    rows, d = x.shape
    ln = op == "layernorm"
    ld = {k: d for k in ("dy", "x", "dx")} | (ld or {})
    off = {k: 0 for k in ("dy", "x", "dx")} | (off or {})
    DY = GuardedRows(torch, dev, dt, rows, d, ld["dy"], off["dy"], dy)
    X = GuardedRows(torch, dev, dt, rows, d, ld["x"], off["x"], x)
    ins = {"dy": (DY, ld["dy"]), "x": (X, ld["x"])}
    DX, lddx = ins[dx_mode] if dx_mode else (GuardedRows(torch, dev, dt, rows, d, ld["dx"], off["dx"]), ld["dx"])
    P0 = GuardedVec(torch, dev, d, po, p0)
    M = GuardedVec(torch, dev, rows, 0, mean) if ln else None
    S = GuardedVec(torch, dev, rows, 0, rstd)
    DG = GuardedVec(torch, dev, d) if param_grads else None
    DB = GuardedVec(torch, dev, d) if (param_grads and ln) else None
    prob = mn.bwd_problem(OPS[op], rows, d, DY.ptr, X.ptr, DX.ptr, P0.ptr, M.ptr if M else None, S.ptr,
                          DG.ptr if DG else None, DB.ptr if DB else None, dtype=dt, lddy=ld["dy"], ldx=ld["x"],
                          lddx=lddx)
    nbytes = mn.mi_norm_bwd_workspace_size(prob)
    assert nbytes >= 0
    WSB = GuardedVec(torch, dev, max(1, (nbytes + 3) // 4), 0, np.full(max(1, (nbytes + 3) // 4), np.nan, np.float32))
    prob.workspace, prob.workspace_bytes = WSB.ptr, nbytes
    stream = torch.cuda.current_stream().cuda_stream
    if expect is not None:
        assert mn.mi_norm_variant_name(mn.mi_norm_bwd_select(prob)) == expect
    if variant is None:
        mn.mi_norm_bwd(prob, stream)
    else:
        mn.mi_norm_bwd_variant(variant, prob, stream)
    torch.cuda.synchronize()
    ref = ref or bwd_ref(op, dt, dy, x, p0, mean, rstd)
    got = DX.rows_host()
    ok, err, ratio = oracle.dx_tolerance_ok(got, ref["dx64"], ref["dx_scale"], FMT.get(dt))
    assert ok, f"dx: max abs err {err:.3e}, err/bound {ratio:.3f}"
    if param_grads:
        pairs = [(DG, "dgamma", "abs_dgamma"), (DB, "dbeta", "abs_dbeta")] if ln else [(DG, "dw", "abs_dw")]
        for buf, key, akey in pairs:
            ok, err, ratio = oracle.colsum_tolerance_ok(buf.host(), ref[key + "64"], ref[akey])
            assert ok, f"{key}: max abs err {err:.3e}, err/bound {ratio:.3f}"
            assert buf.intact(), f"{key}: write outside its range"
    for g, what in ((DY, "dy"), (X, "x"), (DX, "dx")):
        assert g.intact(), f"{what}: write outside its rows"
    for v, what in ((P0, "params"), (M, "mean"), (S, "rstd"), (WSB, "workspace")):
        if v is not None:
            assert v.intact(), f"{what}: write outside its range"
    if dx_mode != "x":
        assert np.array_equal(X.rows_host().view(X.np_bits), np.asarray(x).view(X.np_bits)), "x was modified"
    if dx_mode != "dy":
        assert np.array_equal(DY.rows_host().view(DY.np_bits), np.asarray(dy).view(DY.np_bits)), "dy was modified"


# --- the pages' shapes and patterns, every storage type ------------------------

SHAPES = [(512, 128, "normal"), (512, 128, "zero"), (512, 128, "tiny"), (512, 128, "alternating"),
          (4096, 768, "normal"), (8192, 768, "offset"), (1024, 2048, "offset"), (2048, 4096, "normal"),
          (64, 1, "normal"), (64, 31, "alternating"), (64, 33, "normal"), (64, 127, "offset"),
          (64, 2049, "normal"), (256, 8193, "normal"), (300, 8192, "offset"), (40, 12288, "normal")]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("op", list(OPS))
def test_bwd_shapes(torch_dev, op, dt):
    torch, dev = torch_dev
    for rows, d, pat in SHAPES:
        say(f"bwd {op} dt={dt} [{rows}x{d}] {pat}")
        dy, x, p0, mean, rstd = bwd_inputs(op, dt, rows, d, pat, [32, rows, d])
        run_bwd_case(torch, dev, op, dt, dy, x, p0, mean, rstd)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("op", list(OPS))
def test_bwd_wide_and_streamed(torch_dev, op, dt):
    """Widths at and past the held capacities (the streamed path), strided."""
    torch, dev = torch_dev
    for rows, d in ((7, 16384), (5, 40000), (3, 65537), (600, 16384)):
        say(f"bwd wide {op} dt={dt} [{rows}x{d}]")
        dy, x, p0, mean, rstd = bwd_inputs(op, dt, rows, d, "offset", [33, rows, d])
        run_bwd_case(torch, dev, op, dt, dy, x, p0, mean, rstd, ld={"dy": d + 8, "x": d + 16, "dx": d + 24})


# --- the pipelined loop (rows of several waves) --------------------------------
# Row counts that leave the last step's row slots partly empty, workgroups of
# one step (the prefetch runs past the last row), and odd and even step counts.

PIPELINED = [("layernorm", mn.MI_NORM_F32, 4099, 1536, "lnbwd_4_w2_q3_b8"),
             ("layernorm", mn.MI_NORM_F32, 2051, 2048, "lnbwd_4_w4_q2_b8"),
             ("layernorm", mn.MI_NORM_F32, 1027, 3072, "lnbwd_4_w4_q3_b8"),
             ("layernorm", mn.MI_NORM_F32, 515, 4096, "lnbwd_4_w8_q2_b8"),
             ("layernorm", mn.MI_NORM_F32, 100, 4096, "lnbwd_4_w8_q2_b8"),
             ("rmsnorm", mn.MI_NORM_F32, 4099, 1536, "rmsbwd_4_w2_q3_b8"),
             ("rmsnorm", mn.MI_NORM_F32, 2051, 2048, "rmsbwd_4_w4_q2_b8"),
             ("rmsnorm", mn.MI_NORM_F32, 777, 8192, "rmsbwd_4_w8_q4_b8"),
             ("layernorm", mn.MI_NORM_BF16, 1029, 6144, "lnbwd_bf16_8_w8_q2_b8"),
             ("layernorm", mn.MI_NORM_F16, 1023, 3072, "lnbwd_f16_8_w4_q2_b8"),
             ("rmsnorm", mn.MI_NORM_BF16, 517, 8192, "rmsbwd_bf16_8_w8_q2_b8"),
             ("rmsnorm", mn.MI_NORM_BF16, 30, 4096, "rmsbwd_bf16_8_w4_q2_b8")]


@pytest.mark.parametrize("op,dt,rows,d,name", PIPELINED)
def test_bwd_pipelined_dispatch(torch_dev, op, dt, rows, d, name):
    torch, dev = torch_dev
    say(f"bwd pipelined {op} dt={dt} [{rows}x{d}] {name}")
    dy, x, p0, mean, rstd = bwd_inputs(op, dt, rows, d, "offset", [36, rows, d])
    run_bwd_case(torch, dev, op, dt, dy, x, p0, mean, rstd, expect=name)


# --- every compiled backward variant, forced ----------------------------------

def _bwd_widths(v):
    if v["looped"]:
        return [40000, 776] if v["vec"] > 1 else [40001, 777]
    cap = v["max_d"]
    step = v["vec"]
    return sorted(w for w in {cap, cap - step * max(1, cap // (7 * step)), step} if w >= 1)


def _bwd_layout(v, d):
    if v["needs_aligned"]:
        return dict(ld={"dy": d + 8, "x": d + 16, "dx": d + 24}, off={"dy": 0, "x": 0, "dx": 0}, po=0)
    return dict(ld={"dy": d + 3, "x": d + 1, "dx": d + 5}, off={"dy": 1, "x": 2, "dx": 3}, po=1)


def test_bwd_every_variant(torch_dev):
    torch, dev = torch_dev
    n = 0
    for vid in range(mn.mi_norm_variant_count()):
        v = mn.mi_norm_variant_get_info(vid)
        if v["op"] not in (mn.OP_LAYERNORM_BWD, mn.OP_RMSNORM_BWD):
            continue
        name = mn.mi_norm_variant_name(vid)
        op = "layernorm" if v["op"] == mn.OP_LAYERNORM_BWD else "rmsnorm"
        dt = v["dtype"]
        for d in _bwd_widths(v):
            rows = min(2 * 8 * 512 // max(1, d // 64) + 3, max(3, 400000 // d))
            lay = _bwd_layout(v, d)
            say(f"bwd variant {vid} {name} rows={rows} d={d} {lay}")
            dy, x, p0, mean, rstd = bwd_inputs(op, dt, rows, d, "offset", [34, vid, d])
            run_bwd_case(torch, dev, op, dt, dy, x, p0, mean, rstd, variant=vid, **lay)
            n += 1
    assert n > 0


# --- aliasing, options, edge cases -------------------------------------------

@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("op", list(OPS))
@pytest.mark.parametrize("dx_mode", ["dy", "x"])
def test_bwd_in_place(torch_dev, op, dt, dx_mode):
    torch, dev = torch_dev
    # one-wave rows, pipelined vector rows, pipelined single-element rows, streamed rows
    for rows, d in ((300, 768), (515, 3072), (33, 2049), (4, 40000)):
        say(f"bwd in place {op} dt={dt} dx={dx_mode} [{rows}x{d}]")
        dy, x, p0, mean, rstd = bwd_inputs(op, dt, rows, d, "offset", [35, rows, d])
        ld = d + 8
        run_bwd_case(torch, dev, op, dt, dy, x, p0, mean, rstd, dx_mode=dx_mode,
                     ld={"dy": ld, "x": ld, "dx": ld})


@pytest.mark.parametrize("op", list(OPS))
def test_bwd_without_param_grads_and_zero_rows(torch_dev, op):
    torch, dev = torch_dev
    for rows, d in ((100, 768), (5, 40000)):
        say(f"bwd dx only {op} [{rows}x{d}]")
        dy, x, p0, mean, rstd = bwd_inputs(op, mn.MI_NORM_F32, rows, d, "normal", [36, d])
        run_bwd_case(torch, dev, op, mn.MI_NORM_F32, dy, x, p0, mean, rstd, param_grads=False)
    # no rows: the parameter gradients are zero sums
    say(f"bwd zero rows {op}")
    d = 96
    p0 = wl.make_weight(d, [37])
    dg = torch.full((d,), 7.0, device=dev)
    db = torch.full((d,), 7.0, device=dev)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    one = torch.ones(1, device=dev)
    p = mn.bwd_problem(OPS[op], 0, d, one, one, torch.empty(1, device=dev), torch.from_numpy(p0).to(dev),
                       one if op == "layernorm" else None, one, dg, db if op == "layernorm" else None, ws,
                       ws.numel())
    mn.mi_norm_bwd(p)
    torch.cuda.synchronize()
    assert not bool(dg.any())
    if op == "layernorm":
        assert not bool(db.any())


def test_bwd_stream_ordering_and_repeat(torch_dev):
    """Two calls on a side stream reuse one workspace back to back; the second
    sees its own partial sums only."""
    torch, dev = torch_dev
    rows, d = 4096, 768
    say("bwd stream ordering")
    dy, x, p0, mean, rstd = bwd_inputs("layernorm", mn.MI_NORM_F32, rows, d, "normal", [38])
    dy2 = (dy * np.float32(-2)).astype(np.float32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    X, DY, DY2, G, M, S = t(x), t(dy), t(dy2), t(p0), t(mean), t(rstd)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        dx1, dg1, db1 = mn.layernorm_bwd(DY, X, G, M, S)
        dx2, dg2, db2 = mn.layernorm_bwd(DY2, X, G, M, S)
    torch.cuda.synchronize()
    r1 = oracle.layernorm_bwd(dy, x, p0, mean, rstd)
    r2 = oracle.layernorm_bwd(dy2, x, p0, mean, rstd)
    assert oracle.dx_tolerance_ok(dx1.cpu().numpy(), r1["dx64"], r1["dx_scale"])[0]
    assert oracle.dx_tolerance_ok(dx2.cpu().numpy(), r2["dx64"], r2["dx_scale"])[0]
    assert oracle.colsum_tolerance_ok(dg2.cpu().numpy(), r2["dgamma64"], r2["abs_dgamma"])[0]
    assert oracle.colsum_tolerance_ok(db2.cpu().numpy(), r2["dbeta64"], r2["abs_dbeta"])[0]
    assert oracle.colsum_tolerance_ok(dg1.cpu().numpy(), r1["dgamma64"], r1["abs_dgamma"])[0]


@pytest.mark.parametrize("rows,d", [(8192, 1024), (4099, 3072)])
def test_bwd_deterministic(torch_dev, rows, d):
    """dx and the parameter gradients come out bit for bit the same on every
    call (one-wave rows, and the pipelined loop of rows of several waves)."""
    torch, dev = torch_dev
    say(f"bwd deterministic [{rows}x{d}]")
    dy, x, p0, mean, rstd = bwd_inputs("layernorm", mn.MI_NORM_F32, rows, d, "offset", [39])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    outs = [mn.layernorm_bwd(t(dy), t(x), t(p0), t(mean), t(rstd)) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        for a, b in zip(o, outs[0]):
            assert torch.equal(a, b)


def test_bwd_workspace_reused_across_shapes(torch_dev):
    """One workspace serves calls of several shapes in turn, each matching
    the oracle: nothing a call leaves in the workspace leaks into the next
    one's results (the last call repeats the first shape with new inputs)."""
    torch, dev = torch_dev
    say("bwd one workspace, several shapes")
    cases = [("layernorm", 4096, 768), ("rmsnorm", 3000, 2048), ("layernorm", 2048, 4096),
             ("layernorm", 300, 1024), ("rmsnorm", 4096, 768), ("layernorm", 4096, 768)]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    most = 0
    for op, rows, d in cases:
        # the size depends on the op, shape and which gradients are wanted
        # (non-null), not on the addresses
        p = mn.bwd_problem(OPS[op], rows, d, 0, 0, 0, 0, 0, 0, 256, 256 if op == "layernorm" else None)
        most = max(most, mn.mi_norm_bwd_workspace_size(p))
    WS = torch.full((most,), 0x7F, dtype=torch.uint8, device=dev)   # contents on entry do not matter
    for k, (op, rows, d) in enumerate(cases):
        say(f"  {op} [{rows},{d}]")
        dy, x, p0, mean, rstd = bwd_inputs(op, mn.MI_NORM_F32, rows, d, "offset", [44, k])
        ln = op == "layernorm"
        DY, X, P0, S = t(dy), t(x), t(p0), t(rstd)
        M = t(mean) if ln else None
        DX, DG = torch.empty_like(X), torch.empty(d, device=dev)
        DB = torch.empty(d, device=dev) if ln else None
        p = mn.bwd_problem(OPS[op], rows, d, DY, X, DX, P0, M, S, DG, DB)
        p.workspace, p.workspace_bytes = WS.data_ptr(), most
        mn.mi_norm_bwd(p)
        torch.cuda.synchronize()
        ref = bwd_ref(op, mn.MI_NORM_F32, dy, x, p0, mean, rstd)
        assert oracle.dx_tolerance_ok(DX.cpu().numpy(), ref["dx64"], ref["dx_scale"])[0]
        key = "dgamma" if ln else "dw"
        assert oracle.colsum_tolerance_ok(DG.cpu().numpy(), ref[key + "64"], ref["abs_" + key])[0]
        if ln:
            assert oracle.colsum_tolerance_ok(DB.cpu().numpy(), ref["dbeta64"], ref["abs_dbeta"])[0]


@pytest.mark.parametrize("dt", DTS)
def test_bwd_full_size(torch_dev, dt):
    """[32768, 8192] through the dispatcher: dx on sampled rows and every
    parameter-gradient column against the oracle over all rows."""
    torch, dev = torch_dev
    rows, d = 32768, 8192
    say(f"bwd full size dt={dt}")
    dy, x, p0, mean, rstd = bwd_inputs("layernorm", dt, rows, d, "normal", [40])
    tdt = {mn.MI_NORM_F32: torch.float32, mn.MI_NORM_F16: torch.float16, mn.MI_NORM_BF16: torch.bfloat16}[dt]

    def t(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16)).to(dev).view(tdt) if a.dtype == np.uint16 else torch.from_numpy(a).to(dev)

    dx, dg, db = mn.layernorm_bwd(t(dy), t(x), t(p0), t(mean), t(rstd))
    torch.cuda.synchronize()
    ref = bwd_ref("layernorm", dt, dy, x, p0, mean, rstd)
    sample = np.unique(np.random.default_rng(40).integers(0, rows, 256))
    got = dx[torch.from_numpy(sample).to(dev)].cpu()
    got = got.numpy() if dt == mn.MI_NORM_F32 else got.view(torch.int16).numpy().view(np.uint16)
    assert oracle.dx_tolerance_ok(got, ref["dx64"][sample], ref["dx_scale"][sample], FMT.get(dt))[0]
    ok, err, ratio = oracle.colsum_tolerance_ok(dg.cpu().numpy(), ref["dgamma64"], ref["abs_dgamma"])
    assert ok, f"dgamma: {err:.3e} {ratio:.3f}"
    ok, err, ratio = oracle.colsum_tolerance_ok(db.cpu().numpy(), ref["dbeta64"], ref["abs_dbeta"])
    assert ok, f"dbeta: {err:.3e} {ratio:.3f}"


def test_binding_bwd_16bit_strided_view(torch_dev):
    torch, dev = torch_dev
    say("bwd binding bf16 strided views")
    base_x = torch.randn(200, 1100, device=dev).to(torch.bfloat16)
    base_dy = torch.randn(200, 1000, device=dev).to(torch.bfloat16)
    x, dy = base_x[:, 8:776], base_dy[:, 24:792]
    g = torch.from_numpy(wl.make_affine(768, [41])[0]).to(dev)
    b = torch.zeros(768, device=dev)
    y, mean, rstd = mn.layernorm(x, g, b, wl.EPS, stats=True)
    dx, dg, db = mn.layernorm_bwd(dy, x, g, mean, rstd)
    torch.cuda.synchronize()
    bits = lambda t_: t_.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    ref = oracle.layernorm_bwd16(bits(dy), bits(x), oracle.FMT_BF16, g.cpu().numpy(), mean.cpu().numpy(),
                                 rstd.cpu().numpy())
    assert oracle.dx_tolerance_ok(bits(dx), ref["dx64"], ref["dx_scale"], oracle.FMT_BF16)[0]
    assert oracle.colsum_tolerance_ok(dg.cpu().numpy(), ref["dgamma64"], ref["abs_dgamma"])[0]
    assert oracle.colsum_tolerance_ok(db.cpu().numpy(), ref["dbeta64"], ref["abs_dbeta"])[0]


def test_graph_capture_replays(torch_dev):
    """Forward and backward calls captured in a HIP graph (no allocation or
    memset inside) give the eager results on every replay, with the program's
    own eager work and synchronizations between replays."""
    torch, dev = torch_dev
    rows, d = 2048, 1024
    say("graph capture fwd + bwd")
    x = wl.make_x(rows, d, "offset", [42])
    dy = wl.make_x(rows, d, "normal", [43])
    g, b = wl.make_affine(d, [42, d])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    X, DY, G, B = t(x), t(dy), t(g), t(b)
    Y, M, S = torch.empty_like(X), torch.empty(rows, device=dev), torch.empty(rows, device=dev)
    DX, DG, DB = torch.empty_like(X), torch.empty(d, device=dev), torch.empty(d, device=dev)
    p = mn.bwd_problem(mn.OP_LAYERNORM, rows, d, DY, X, DX, G, M, S, DG, DB)
    nbytes = mn.mi_norm_bwd_workspace_size(p)
    WS = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    p.workspace, p.workspace_bytes = WS.data_ptr(), nbytes
    s = torch.cuda.Stream()
    torch.cuda.synchronize()

    def step(stream):
        mn.mi_layernorm_fwd(X, G, B, Y, rows, d, wl.EPS, M, S, stream=stream)
        mn.mi_norm_bwd(p, stream)

    with torch.cuda.stream(s):
        step(s.cuda_stream)
    torch.cuda.synchronize()
    eager = [a.clone() for a in (Y, M, S, DX, DG, DB)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step(s.cuda_stream)
    for k in range(4):
        for a in (Y, M, S, DX, DG, DB):
            a.fill_(float("nan"))           # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, e in zip((Y, M, S, DX, DG, DB), eager):
            assert torch.equal(a, e), f"replay {k} differs from the eager call"
