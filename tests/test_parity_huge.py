"""GPU parity at the largest sizes: tensors past 2^31 and 2^32 elements, so
every row offset and element index must be 64-bit.  Inputs are drawn on the
device (seeded torch generator); sampled rows, the first and the last
included, are checked against the float64 oracle, and every row's statistics
must be finite."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import row_wise_normalization_layernorm_amd as mn
from row_wise_normalization_layernorm_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    mn.lib()
    return torch, torch.device("cuda:0")


def _sample(rows, seed):
    s = np.unique(np.random.default_rng(seed).integers(0, rows, 96))
    return np.unique(np.concatenate([[0, 1, rows - 2, rows - 1], s]))


def _rows(torch, t, idx, bits16=False):
    a = t[torch.from_numpy(idx).to(t.device)].cpu()
    return a.view(torch.int16).numpy().view(np.uint16) if bits16 else a.numpy()


def test_layernorm_past_2e31_elements(torch_dev):
    torch, dev = torch_dev
    rows, d = 270001, 8192                      # 2.21e9 elements, 8.8 GB per tensor
    print(f"huge layernorm f32 [{rows}x{d}]", flush=True)
    gen = torch.Generator(device=dev).manual_seed(51)
    x = torch.randn(rows, d, device=dev, generator=gen)
    g, b = (torch.from_numpy(a).to(dev) for a in wl.make_affine(d, [51, d]))
    y, mean, rstd = mn.layernorm(x, g, b, wl.EPS, stats=True)
    torch.cuda.synchronize()
    idx = _sample(rows, 51)
    ry, rm, rr, _, _ = oracle.layernorm(_rows(torch, x, idx), g.cpu().numpy(), b.cpu().numpy(), wl.EPS)
    for got, want, what in ((_rows(torch, y, idx), ry, "y"), (mean.cpu().numpy()[idx], rm, "mean"),
                            (rstd.cpu().numpy()[idx], rr, "rstd")):
        ok, err, ratio = oracle.tolerance_ok(got, want)
        assert ok, f"{what}: max abs err {err:.3e}, err/bound {ratio:.3f}"
    assert bool(torch.isfinite(mean).all()) and bool(torch.isfinite(rstd).all())
    del x, y, mean, rstd
    torch.cuda.empty_cache()


def test_fused_bf16_past_2e32_elements(torch_dev):
    torch, dev = torch_dev
    rows, d = 540001, 8192                      # 4.42e9 elements, 8.8 GB per tensor, four tensors
    print(f"huge add_rmsnorm bf16 [{rows}x{d}]", flush=True)
    gen = torch.Generator(device=dev).manual_seed(52)
    x = torch.randn(rows, d, device=dev, dtype=torch.bfloat16, generator=gen)
    r = torch.randn(rows, d, device=dev, dtype=torch.bfloat16, generator=gen)
    w = torch.from_numpy(wl.make_weight(d, [52, d])).to(dev)
    y, h, rstd = mn.add_rmsnorm(x, r, w, wl.EPS, stats=True)
    torch.cuda.synchronize()
    idx = _sample(rows, 52)
    _, y64, hh, s = oracle.add_rmsnorm16(_rows(torch, x, idx, True), _rows(torch, r, idx, True), oracle.FMT_BF16,
                                         w.cpu().numpy(), wl.EPS)
    ok, err, ratio = oracle.tolerance_ok16(_rows(torch, y, idx, True), y64, oracle.FMT_BF16)
    assert ok, f"y: max abs err {err:.3e}, err/bound {ratio:.3f}"
    assert np.array_equal(_rows(torch, h, idx, True), hh.view(np.uint16)), "h != x + r"
    assert oracle.tolerance_ok(rstd.cpu().numpy()[idx], s)[0]
    assert bool(torch.isfinite(rstd).all())
    del x, r, y, h, rstd
    torch.cuda.empty_cache()


def test_layernorm_backward_past_2e31_elements(torch_dev):
    torch, dev = torch_dev
    rows, d = 270001, 8192
    print(f"huge layernorm backward f32 [{rows}x{d}]", flush=True)
    gen = torch.Generator(device=dev).manual_seed(53)
    x = torch.randn(rows, d, device=dev, generator=gen)
    dy = torch.randn(rows, d, device=dev, generator=gen)
    g, b = (torch.from_numpy(a).to(dev) for a in wl.make_affine(d, [53, d]))
    _, mean, rstd = mn.layernorm(x, g, b, wl.EPS, stats=True)
    dx, dg, db = mn.layernorm_bwd(dy, x, g, mean, rstd)
    torch.cuda.synchronize()
    idx = _sample(rows, 53)
    ref = oracle.layernorm_bwd(_rows(torch, dy, idx), _rows(torch, x, idx), g.cpu().numpy(),
                               mean.cpu().numpy()[idx], rstd.cpu().numpy()[idx])
    ok, err, ratio = oracle.dx_tolerance_ok(_rows(torch, dx, idx), ref["dx64"], ref["dx_scale"])
    assert ok, f"dx: max abs err {err:.3e}, err/bound {ratio:.3f}"
    # the parameter gradients sum over every row.  Column j's sums need only
    # column j of x and dy and every row's mean/rstd, so the oracle takes
    # sampled columns whole (its dx for such narrowed rows is not used).
    cols = np.unique(np.concatenate([[0, d - 1], np.random.default_rng(54).integers(0, d, 14)]))
    ct = torch.from_numpy(cols).to(dev)
    refc = oracle.layernorm_bwd(np.ascontiguousarray(dy[:, ct].cpu().numpy()),
                                np.ascontiguousarray(x[:, ct].cpu().numpy()), g.cpu().numpy()[cols],
                                mean.cpu().numpy(), rstd.cpu().numpy())
    for got, key in ((dg.cpu().numpy()[cols], "dgamma"), (db.cpu().numpy()[cols], "dbeta")):
        ok, err, ratio = oracle.colsum_tolerance_ok(got, refc[key + "64"], refc["abs_" + key])
        assert ok, f"{key}: max abs err {err:.3e}, err/bound {ratio:.3f}"
    del x, dy, dx, mean, rstd
    torch.cuda.empty_cache()

