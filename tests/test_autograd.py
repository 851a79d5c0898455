"""GPU tests of the differentiable layer (row_wise_normalization_layernorm_amd.autograd):
a training-style forward and backward through torch autograd runs the
library's forward and backward kernels, checked against the float64 oracle;
and the binding's calls on side streams (torch stream or raw handle) give
the default stream's results."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import row_wise_normalization_layernorm_amd as mn
from row_wise_normalization_layernorm_amd import workloads as wl

pytestmark = pytest.mark.gpu

FMT = {"f32": None, "bf16": oracle.FMT_BF16}


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    mn.lib()
    return torch, torch.device("cuda:0")


def _device(torch, dev, a, fmt):
    if fmt is None:
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def _host(t, fmt):
    import torch
    a = t.detach().cpu()
    return a.numpy() if fmt is None else a.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("op", ["layernorm", "rmsnorm"])
def test_module_forward_backward_match_the_oracle(torch_dev, op, kind):
    torch, dev = torch_dev
    fmt = FMT[kind]
    b0, b1, d = 3, 97, 768
    print(f"autograd {op} {kind} [{b0}x{b1}x{d}]", flush=True)
    x = wl.make_x(b0 * b1, d, "offset", [41, d])
    dy = wl.make_x(b0 * b1, d, "normal", [42, d])
    if fmt:
        x, dy = wl.quantize16(x, fmt), wl.quantize16(dy, fmt)
    ln = op == "layernorm"
    m = (mn.LayerNorm(d, device=dev) if ln else mn.RMSNorm(d, device=dev))
    with torch.no_grad():
        if ln:
            g, bt = wl.make_affine(d, [43, d])
            m.weight.copy_(torch.from_numpy(g)), m.bias.copy_(torch.from_numpy(bt))
        else:
            g = wl.make_weight(d, [43, d])
            m.weight.copy_(torch.from_numpy(g))
    xt = _device(torch, dev, x, fmt).reshape(b0, b1, d).requires_grad_(True)
    y = m(xt)
    y.backward(_device(torch, dev, dy, fmt).reshape(b0, b1, d))
    torch.cuda.synchronize()
    assert y.shape == xt.shape and y.dtype == xt.dtype and xt.grad.dtype == xt.dtype

    # forward
    got_y = _host(y, fmt).reshape(b0 * b1, d)
    if ln:
        fw = oracle.layernorm16(x, fmt, g, bt, wl.EPS) if fmt else oracle.layernorm(x, g, bt, wl.EPS)
        mean, rstd = (fw[2], fw[3]) if fmt else (fw[1], fw[2])
    else:
        fw = oracle.rmsnorm16(x, fmt, g, wl.EPS) if fmt else oracle.rmsnorm(x, g, wl.EPS)
        mean, rstd = None, (fw[2] if fmt else fw[1])
    ok = oracle.tolerance_ok16(got_y, fw[1], fmt)[0] if fmt else oracle.tolerance_ok(got_y, fw[0])[0]
    assert ok, "y"
    # backward, from the oracle's own statistics
    if ln:
        ref = oracle.layernorm_bwd16(dy, x, fmt, g, mean, rstd) if fmt else oracle.layernorm_bwd(dy, x, g, mean, rstd)
        grads = [(m.weight.grad, "dgamma"), (m.bias.grad, "dbeta")]
    else:
        ref = oracle.rmsnorm_bwd16(dy, x, fmt, g, rstd) if fmt else oracle.rmsnorm_bwd(dy, x, g, rstd)
        grads = [(m.weight.grad, "dw")]
    ok, err, ratio = oracle.dx_tolerance_ok(np.ascontiguousarray(_host(xt.grad, fmt).reshape(b0 * b1, d)),
                                            ref["dx64"], ref["dx_scale"], fmt)
    assert ok, f"dx: max abs err {err:.3e}, err/bound {ratio:.3f}"
    for t, key in grads:
        ok, err, ratio = oracle.colsum_tolerance_ok(t.detach().cpu().numpy(), ref[key + "64"], ref["abs_" + key])
        assert ok, f"{key}: max abs err {err:.3e}, err/bound {ratio:.3f}"


def test_frozen_parameters_and_strided_input(torch_dev):
    """No parameter gradients when the parameters do not require them, and a
    column slice (strided rows) as input."""
    torch, dev = torch_dev
    x = torch.randn(64, 1024, device=dev)[:, :768].requires_grad_(True)
    w = torch.ones(768, device=dev)
    y = mn.rms_norm(x, w)
    y.sum().backward()
    torch.cuda.synchronize()
    assert w.grad is None and x.grad.shape == x.shape
    # d(sum y)/dx for RMSNorm with w = 1: rstd * (1 - xhat * mean(xhat)), xhat = x * rstd
    xd = x.detach().double()
    rs = 1.0 / torch.sqrt((xd * xd).mean(-1, keepdim=True) + 1e-5)
    xh = xd * rs
    want = rs * (1.0 - xh * xh.mean(-1, keepdim=True))
    assert torch.allclose(x.grad.double(), want, atol=1e-5, rtol=1e-4)


def test_side_streams_give_the_default_streams_results(torch_dev):
    torch, dev = torch_dev
    x = torch.randn(300, 768, device=dev)
    dy = torch.randn(300, 768, device=dev)
    g = torch.randn(768, device=dev) * 0.1 + 1
    b = torch.randn(768, device=dev) * 0.1
    y0, m0, r0 = mn.layernorm(x, g, b, stats=True)
    b0 = mn.layernorm_bwd(dy, x, g, m0, r0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream())
    for s in (side, side.cuda_stream):
        y1, m1, r1 = mn.layernorm(x, g, b, stats=True, stream=s)
        b1 = mn.layernorm_bwd(dy, x, g, m1, r1, stream=s)
        side.synchronize()
        for a, c in zip((y0, m0, r0) + tuple(b0), (y1, m1, r1) + tuple(b1)):
            assert torch.equal(a, c)


def test_expanded_upstream_gradient_and_inputs(torch_dev):
    """A loss that sums over rows hands the backward an upstream gradient
    whose rows repeat (stride 0); the binding copies such an input rather
    than pass a row stride the kernels would read as d.  An expanded x in
    the forward is copied the same way, and an expanded output is refused."""
    torch, dev = torch_dev
    print("autograd expanded dy [256x768]", flush=True)
    gen = torch.Generator(device="cpu").manual_seed(31)
    x = (torch.randn(256, 768, generator=gen) * 3 + 0.5).to(dev).requires_grad_(True)
    g = (torch.randn(768, generator=gen) * 0.1 + 1).to(dev).requires_grad_(True)
    b = (torch.randn(768, generator=gen) * 0.1).to(dev).requires_grad_(True)
    y = mn.layer_norm(x, g, b)
    y.sum(0).pow(2).sum().backward()
    torch.cuda.synchronize()
    # the upstream gradient autograd handed the backward: 2 * y.sum(0) for
    # every row (stride 0), from the same forward kernel's y
    y2, mean, rstd = mn.layernorm(x.detach(), g.detach(), b.detach(), stats=True)
    assert torch.equal(y2, y.detach())
    dy = (2 * y2.sum(0)).expand_as(y2)
    assert dy.stride(0) == 0
    ref = oracle.layernorm_bwd(dy.contiguous().cpu().numpy(), x.detach().cpu().numpy(), g.detach().cpu().numpy(),
                               mean.cpu().numpy(), rstd.cpu().numpy())
    ok, err, ratio = oracle.dx_tolerance_ok(x.grad.cpu().numpy(), ref["dx64"], ref["dx_scale"])
    assert ok, (err, ratio)
    for got, key in ((g.grad, "dgamma"), (b.grad, "dbeta")):
        ok, err, ratio = oracle.colsum_tolerance_ok(got.cpu().numpy(), ref[key + "64"], ref["abs_" + key])
        assert ok, (key, err, ratio)
    # the direct call with the expanded gradient gives autograd's bits
    dx, dg, db = mn.layernorm_bwd(dy, x.detach(), g.detach(), mean, rstd)
    assert torch.equal(dx, x.grad) and torch.equal(dg, g.grad) and torch.equal(db, b.grad)

    row = torch.randn(1, 768, device=dev)
    xe = row.expand(64, 768)
    ye = mn.layernorm(xe, g.detach(), b.detach())
    assert torch.equal(ye, mn.layernorm(xe.contiguous(), g.detach(), b.detach()))
    with pytest.raises(ValueError):
        mn.layernorm(torch.randn(64, 768, device=dev), g.detach(), b.detach(), out=torch.empty(1, 768, device=dev).expand(64, 768))
