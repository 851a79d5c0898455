"""GPU test of mi_norm_bwd_noalloc, the backward entry point that allocates
nothing: called through the C ABI, its outputs must equal those of
mi_norm_bwd with a caller-owned workspace, bit for bit (the same kernels in
the same order), and lie within the oracle's acceptance bounds; on two calls
in a row, the second with a smaller input (the scratch array keeps the first
call's contents), for LayerNorm and RMSNorm, float32 and bfloat16 rows.
Problems that need more scratch than the array holds, or that pass a
workspace, are refused before any launch."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import row_wise_normalization_layernorm_amd as mn
from row_wise_normalization_layernorm_amd import workloads as wl

pytestmark = pytest.mark.gpu

FMT = {mn.MI_NORM_F32: None, mn.MI_NORM_BF16: oracle.FMT_BF16}


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    mn.lib()
    return torch, torch.device("cuda:0")


def _case(torch, dev, op, dt, rows, d, seed):
    ln = op == mn.OP_LAYERNORM
    fmt = FMT[dt]
    x = wl.make_x(rows, d, "offset", seed)
    dy = wl.make_x(rows, d, "normal", [61] + seed)
    p0 = wl.make_affine(d, [61, d])[0] if ln else wl.make_weight(d, [61, d])
    if fmt is not None:
        x, dy = wl.quantize16(x, fmt), wl.quantize16(dy, fmt)
        xw = oracle.widen16(x, fmt)
    else:
        xw = x
    if ln:
        _, mean, rstd, _, _ = oracle.layernorm(xw, p0, np.zeros(d, np.float32), wl.EPS)
    else:
        _, rstd, _ = oracle.rmsnorm(xw, p0, wl.EPS)
        mean = None

    def dev_rows(a):
        a = np.ascontiguousarray(a)
        if fmt is None:
            return torch.from_numpy(a).to(dev)
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    ins = dict(dy=dev_rows(dy), x=dev_rows(x), p0=t(p0), mean=t(mean) if ln else None, rstd=t(rstd))
    ref = ((oracle.layernorm_bwd16(dy, x, fmt, p0, mean, rstd) if ln else oracle.rmsnorm_bwd16(dy, x, fmt, p0, rstd))
           if fmt is not None else
           (oracle.layernorm_bwd(dy, x, p0, mean, rstd) if ln else oracle.rmsnorm_bwd(dy, x, p0, rstd)))
    return ins, ref


def _outputs(torch, dev, ins, ln, dt):
    dx = torch.empty_like(ins["x"])
    dg = torch.full((ins["x"].shape[1],), float("nan"), device=dev)
    db = torch.full_like(dg, float("nan")) if ln else None
    return dx, dg, db


def _problem(op, dt, ins, outs, ws=None, ws_bytes=0):
    rows, d = ins["x"].shape
    dx, dg, db = outs
    return mn.bwd_problem(op, rows, d, ins["dy"], ins["x"], dx, ins["p0"], ins["mean"], ins["rstd"], dg, db,
                          ws, ws_bytes, dtype=dt)


def _bits(t):
    import torch
    a = t.cpu()
    return a.view(torch.int16).numpy() if a.dtype == torch.bfloat16 else a.numpy().view(np.int32)


@pytest.mark.parametrize("dt", [pytest.param(mn.MI_NORM_F32, id="f32"), pytest.param(mn.MI_NORM_BF16, id="bf16")])
@pytest.mark.parametrize("op", [pytest.param(mn.OP_LAYERNORM, id="layernorm"),
                                pytest.param(mn.OP_RMSNORM, id="rmsnorm")])
def test_noalloc_equals_the_workspace_call(torch_dev, op, dt):
    torch, dev = torch_dev
    ln = op == mn.OP_LAYERNORM
    # two calls in a row; the second is smaller and runs over what the first left
    for k, (rows, d) in enumerate(((4096, 768), (1000, 512))):
        print(f"noalloc op={op} dt={dt} [{rows},{d}]", flush=True)
        ins, ref = _case(torch, dev, op, dt, rows, d, [60, k, op, dt])
        ref_outs = _outputs(torch, dev, ins, ln, dt)
        p = _problem(op, dt, ins, ref_outs)
        nbytes = mn.mi_norm_bwd_workspace_size(p)
        assert 0 < nbytes <= mn.mi_norm_bwd_noalloc_limit()
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        p.workspace, p.workspace_bytes = ws.data_ptr(), nbytes
        mn.mi_norm_bwd(p)
        outs = _outputs(torch, dev, ins, ln, dt)
        mn.mi_norm_bwd_noalloc(_problem(op, dt, ins, outs))
        torch.cuda.synchronize()
        for a, b in zip(outs, ref_outs):
            if a is not None:
                assert np.array_equal(_bits(a), _bits(b))
        fmt = FMT[dt]
        dxh = _bits(outs[0]).view(np.uint16) if fmt is not None else outs[0].cpu().numpy()
        assert oracle.dx_tolerance_ok(dxh, ref["dx64"], ref["dx_scale"], fmt)[0]
        keys = [("dgamma", outs[1]), ("dbeta", outs[2])] if ln else [("dw", outs[1])]
        for key, t in keys:
            assert oracle.colsum_tolerance_ok(t.cpu().numpy(), ref[key + "64"], ref["abs_" + key])[0]


def test_noalloc_refuses_what_it_cannot_hold(torch_dev):
    torch, dev = torch_dev
    print("noalloc refusals", flush=True)
    limit = mn.mi_norm_bwd_noalloc_limit()
    assert limit == 32 << 20
    x = torch.zeros(8, 8192, device=dev)
    dy, dx = torch.zeros_like(x), torch.empty_like(x)
    g, m, s = torch.ones(8192, device=dev), torch.zeros(8, device=dev), torch.ones(8, device=dev)
    dg, db = torch.empty(8192, device=dev), torch.empty(8192, device=dev)
    fits = mn.bwd_problem(mn.OP_LAYERNORM, 8, 8192, dy, x, dx, g, m, s, dg, db)
    assert mn.mi_norm_bwd_workspace_size(fits) <= limit
    # a caller's workspace is not taken
    ws = torch.empty(mn.mi_norm_bwd_workspace_size(fits), dtype=torch.uint8, device=dev)
    with pytest.raises(mn.MiNormError) as e:
        mn.mi_norm_bwd_noalloc(mn.bwd_problem(mn.OP_LAYERNORM, 8, 8192, dy, x, dx, g, m, s, dg, db, ws,
                                              ws.numel()))
    assert e.value.status == mn.MI_NORM_ERR_INVALID
    # 2^21 + 1 rows of 8192: more workspace than the array holds (sizes only; nothing launched)
    big = mn.bwd_problem(mn.OP_LAYERNORM, (1 << 21) + 1, 8192, dy, x, dx, g, m, s, dg, db)
    assert mn.mi_norm_bwd_workspace_size(big) > limit
    with pytest.raises(mn.MiNormError) as e:
        mn.mi_norm_bwd_noalloc(big)
    assert e.value.status == mn.MI_NORM_ERR_INVALID
    torch.cuda.synchronize()
