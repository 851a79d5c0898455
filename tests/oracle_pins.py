"""Checks that pin the CPU oracle to facts outside itself.

Each ``check_*`` takes an oracle library handle (``oracle.load(path)``) and
raises AssertionError when the oracle disagrees with:

* exact rational brute force on tiny inputs (Fraction statistics, 60-digit
  Decimal root), which is the definition evaluated without rounding;
* torch's float64 CPU LayerNorm / RMSNorm library routines, an independent
  implementation of the same definitions;
* closed forms (zero rows, width 1, alternating +-1, constant rows);
* invariants (shift and power-of-two scale invariance, column and row
  permutation equivariance, unit-affine output moments, in-place equality).

The definitions pinned are the statistics equation of "Rewriting the layer
norm and matmul kernels" (section "A reduction has to meet somewhere") with a
per-column scale and bias and eps inside the root, and the RMSNorm equation of
"RMSNorm on an RTX 5070" (section "The operator and the change").

tests/test_oracle_pins.py runs every check on the shipped oracle;
tests/test_negative_controls.py runs them on builds with a planted mistake
and requires each mistake to be caught.
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

import oracle
from row_wise_normalization_layernorm_amd import workloads as wl

EPS32 = np.float32(wl.EPS)


# ----------------------------------------------------------------------------
# small helpers (no normalization arithmetic beyond the exact brute force)

def _ulps(a, b) -> np.ndarray:
    """Distance in float32 units in the last place between arrays a and b."""
    a = np.asarray(a, np.float32).astype(np.float64)
    b = np.asarray(b, np.float32).astype(np.float64)
    scale = np.spacing(np.maximum(np.abs(a), np.abs(b)).astype(np.float32)).astype(np.float64)
    scale = np.maximum(scale, np.float64(np.finfo(np.float32).smallest_subnormal))
    return np.abs(a - b) / scale


def _assert_ulps(got, ref, n: float, what: str):
    u = _ulps(got, ref)
    assert np.all(np.isfinite(np.asarray(got, np.float64))), f"{what}: non-finite output"
    assert float(u.max(initial=0.0)) <= n, f"{what}: {float(u.max())} ulp > {n}"


def _dec(f: Fraction) -> Decimal:
    return Decimal(f.numerator) / Decimal(f.denominator)


def _rng(seed):
    return np.random.default_rng(seed)


def _ln(lib, x, g, b, eps=EPS32):
    return oracle.layernorm(x, g, b, float(eps), lib=lib)


def _rms(lib, x, w, eps=EPS32):
    return oracle.rmsnorm(x, w, float(eps), lib=lib)


# ----------------------------------------------------------------------------
# exact brute force

def _exact_ln_row(xrow, g, b, eps):
    getcontext().prec = 60
    xs = [Fraction(float(v)) for v in xrow]
    d = len(xs)
    mu = sum(xs, Fraction(0)) / d
    var = sum(((v - mu) ** 2 for v in xs), Fraction(0)) / d
    rho = 1 / (_dec(var) + _dec(Fraction(float(eps)))).sqrt()
    ys = [_dec(v - mu) * rho * Decimal(float(gj)) + Decimal(float(bj))
          for v, gj, bj in zip(xs, g, b)]
    return mu, var, rho, ys


def _exact_rms_row(xrow, w, eps):
    getcontext().prec = 60
    xs = [Fraction(float(v)) for v in xrow]
    ms = sum((v * v for v in xs), Fraction(0)) / len(xs)
    rho = 1 / (_dec(ms) + _dec(Fraction(float(eps)))).sqrt()
    ys = [_dec(v) * Decimal(float(wj)) * rho for v, wj in zip(xs, w)]
    return ms, rho, ys


def check_ln_bruteforce(lib):
    for d in (1, 2, 3, 5, 8):
        rng = _rng([11, d])
        rows = 6
        x = rng.standard_normal((rows, d)).astype(np.float32)
        x[0] = (x[0].astype(np.float64) * 3 + 0.5).astype(np.float32)
        g = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
        b = (0.1 * rng.standard_normal(d)).astype(np.float32)
        y, mean, rstd, mean64, var64 = _ln(lib, x, g, b)
        for i in range(rows):
            mu, var, rho, ys = _exact_ln_row(x[i], g, b, EPS32)
            scale = float(np.abs(x[i]).max()) + 1e-30
            assert abs(mean64[i] - float(mu)) <= 1e-14 * scale, ("mean64", d, i)
            assert abs(var64[i] - float(var)) <= 1e-13 * scale * scale, ("var64", d, i)
            yex = np.array([float(t) for t in ys], np.float32)
            # float64 evaluation then one rounding: within 1 ulp of the exact
            # result, plus the float64 cancellation floor near zero outputs
            err = np.abs(y[i].astype(np.float64) - np.array([float(t) for t in ys]))
            lim = np.spacing(np.abs(yex)).astype(np.float64) + 1e-14
            assert np.all(err <= lim), ("y", d, i, float(err.max()))
            _assert_ulps(mean[i], np.float32(float(mu)), 1, f"mean d={d}")
            _assert_ulps(rstd[i], np.float32(float(rho)), 1, f"rstd d={d}")


def check_rms_bruteforce(lib):
    for d in (1, 2, 3, 5, 8):
        rng = _rng([12, d])
        rows = 6
        x = rng.standard_normal((rows, d)).astype(np.float32)
        w = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
        y, rstd, ms64 = _rms(lib, x, w)
        for i in range(rows):
            ms, rho, ys = _exact_rms_row(x[i], w, EPS32)
            assert abs(ms64[i] - float(ms)) <= 1e-14 * float(ms) + 1e-300, ("ms64", d, i)
            yex = np.array([float(t) for t in ys], np.float32)
            _assert_ulps(y[i], yex, 1, f"rms y d={d}")
            _assert_ulps(rstd[i], np.float32(float(rho)), 1, f"rms rstd d={d}")


# ----------------------------------------------------------------------------
# independent library implementation (torch float64 on the CPU)

def check_ln_vs_torch(lib):
    import torch
    for rows, d, pat in ((64, 1, "normal"), (37, 7, "offset"), (64, 128, "normal"),
                         (17, 1000, "offset"), (9, 4096, "tiny"), (33, 33, "alternating")):
        x = wl.make_x(rows, d, pat, [13, rows, d])
        g, b = wl.make_affine(d, [13, d])
        y, mean, rstd, mean64, var64 = _ln(lib, x, g, b)
        ty, tmean, trstd = torch.native_layer_norm(
            torch.from_numpy(x).double(), (d,), torch.from_numpy(g).double(),
            torch.from_numpy(b).double(), float(EPS32))
        _assert_ulps(y, ty.numpy().astype(np.float32), 1, f"ln vs torch y {rows}x{d}")
        np.testing.assert_allclose(mean64, tmean.reshape(-1).numpy(), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(1.0 / np.sqrt(var64 + float(EPS32)), trstd.reshape(-1).numpy(),
                                   rtol=1e-12)
        _assert_ulps(rstd, trstd.reshape(-1).numpy().astype(np.float32), 1, "ln vs torch rstd")
        _assert_ulps(mean, tmean.reshape(-1).numpy().astype(np.float32), 1, "ln vs torch mean")


def check_rms_vs_torch(lib):
    import torch
    import torch.nn.functional as F
    for rows, d, pat in ((64, 1, "normal"), (31, 31, "normal"), (64, 128, "tiny"),
                         (8, 8193, "normal"), (16, 4096, "alternating")):
        x = wl.make_x(rows, d, pat, [14, rows, d])
        w = wl.make_weight(d, [14, d])
        y, rstd, ms64 = _rms(lib, x, w)
        ty = F.rms_norm(torch.from_numpy(x).double(), (d,), torch.from_numpy(w).double(),
                        eps=float(EPS32))
        _assert_ulps(y, ty.numpy().astype(np.float32), 1, f"rms vs torch {rows}x{d}")
        tms = (torch.from_numpy(x).double() ** 2).mean(dim=1).numpy()
        np.testing.assert_allclose(ms64, tms, rtol=1e-12, atol=1e-300)


# ----------------------------------------------------------------------------
# closed forms

def check_ln_closed_forms(lib):
    inv_sqrt_eps = np.float32(1.0 / math.sqrt(float(EPS32)))
    # zero rows: x - mu = 0 exactly, so y is beta bit for bit
    d = 257
    g, b = wl.make_affine(d, [15, d])
    x = np.zeros((5, d), np.float32)
    y, mean, rstd, _, _ = _ln(lib, x, g, b)
    assert np.array_equal(y, np.broadcast_to(b, y.shape)), "zero rows: y != beta"
    assert np.all(mean == 0), "zero rows: mean != 0"
    _assert_ulps(rstd, np.full(5, inv_sqrt_eps), 1, "zero rows: rstd != 1/sqrt(eps)")
    # width 1: the single element is its own mean
    x = wl.make_x(16, 1, "normal", [15, 1])
    g1, b1 = wl.make_affine(1, [15, 1])
    y, mean, rstd, _, _ = _ln(lib, x, g1, b1)
    assert np.array_equal(y, np.broadcast_to(b1, y.shape)), "width 1: y != beta"
    assert np.array_equal(mean, x[:, 0]), "width 1: mean != x"
    _assert_ulps(rstd, np.full(16, inv_sqrt_eps), 1, "width 1: rstd")
    # constant rows (dyadic value, exact sum): y == beta
    x = np.full((3, 96), 0.75, np.float32)
    g96, b96 = wl.make_affine(96, [15, 96])
    y, mean, _, _, _ = _ln(lib, x, g96, b96)
    assert np.array_equal(y, np.broadcast_to(b96, y.shape)), "constant rows: y != beta"
    assert np.all(mean == np.float32(0.75))
    # alternating +-1 with p plus and m minus per row: mu = (p-m)/d, var = 1 - mu^2
    for d in (2, 128, 31, 33, 127):
        x = wl.make_x(4, d, "alternating")
        g, b = wl.make_affine(d, [15, 2, d])
        y, mean, rstd, _, var64 = _ln(lib, x, g, b)
        for i in range(4):
            p = int(np.sum(x[i] > 0))
            m = d - p
            mu = (p - m) / d
            var = 1.0 - mu * mu
            rho = 1.0 / math.sqrt(var + float(EPS32))
            assert abs(var64[i] - var) <= 1e-13, ("alt var", d, i)  # float64 rounding of mu
            want = ((x[i].astype(np.float64) - mu) * rho * g + b).astype(np.float32)
            _assert_ulps(y[i], want, 1, f"alternating d={d}")
            _assert_ulps(rstd[i], np.float32(rho), 1, f"alternating rstd d={d}")


def check_rms_closed_forms(lib):
    d = 129
    w = wl.make_weight(d, [16, d])
    y, rstd, _ = _rms(lib, np.zeros((4, d), np.float32), w)
    assert np.all(y == 0), "zero rows: y != 0"
    _assert_ulps(rstd, np.full(4, np.float32(1 / math.sqrt(float(EPS32)))), 1, "zero rstd")
    # width 1: y = x w / sqrt(x^2 + eps)
    x = wl.make_x(32, 1, "normal", [16, 1])
    w1 = wl.make_weight(1, [16, 1])
    y, _, _ = _rms(lib, x, w1)
    xd = x[:, 0].astype(np.float64)
    want = (xd * float(w1[0]) / np.sqrt(xd * xd + float(EPS32))).astype(np.float32)
    _assert_ulps(y[:, 0], want, 1, "rms width 1")
    # alternating: mean square is exactly 1
    for d in (31, 128):
        x = wl.make_x(3, d, "alternating")
        w = wl.make_weight(d, [16, 2, d])
        y, rstd, ms64 = _rms(lib, x, w)
        assert np.all(ms64 == 1.0), "alternating mean square != 1"
        want = (x.astype(np.float64) * w / math.sqrt(1.0 + float(EPS32))).astype(np.float32)
        _assert_ulps(y, want, 1, f"rms alternating d={d}")


# ----------------------------------------------------------------------------
# invariants

def _dyadic(rows, d, seed):
    """Values k/256 with |k| < 2^10: sums of up to 2^20 of them stay exact in float64."""
    k = _rng(seed).integers(-1023, 1024, size=(rows, d))
    return (k / 256.0).astype(np.float32)


def check_ln_invariants(lib):
    rows, d = 12, 256  # power-of-two width: mu = s/d is exact, so every step is exact
    x = _dyadic(rows, d, [17, 1])
    g, b = wl.make_affine(d, [17, 2])
    y0, m0, r0, mu0, var0 = _ln(lib, x, g, b)
    # shift invariance: x + 8 is exact, every float64 step is exact, y is identical
    y1, m1, r1, _, _ = _ln(lib, (x + np.float32(8.0)).astype(np.float32), g, b)
    assert np.array_equal(y0, y1), "LN(x + c) != LN(x)"
    assert np.array_equal(r0, r1), "rstd changed under a shift"
    assert np.allclose(m1, m0 + 8.0, rtol=0, atol=1e-6), "mean did not shift"
    # power-of-two scale: LN_eps(2x) == LN_{eps/4}(x) bit for bit
    y2, _, _, _, _ = _ln(lib, (2 * x).astype(np.float32), g, b, EPS32)
    y3, _, _, _, _ = _ln(lib, x, g, b, np.float32(EPS32 / 4))
    assert np.array_equal(y2, y3), "LN_eps(2x) != LN_eps/4(x)"
    # row permutation: rows are independent
    perm = _rng([17, 3]).permutation(rows)
    yp, _, _, _, _ = _ln(lib, x[perm], g, b)
    assert np.array_equal(yp, y0[perm]), "row permutation"
    # column permutation: every column keeps its own gamma/beta (sum order changes)
    xr = wl.make_x(rows, d, "offset", [17, 4])
    yr, _, _, _, _ = _ln(lib, xr, g, b)
    cp = _rng([17, 5]).permutation(d)
    yc, _, _, _, _ = _ln(lib, np.ascontiguousarray(xr[:, cp]), g[cp], b[cp])
    _assert_ulps(yc, yr[:, cp], 1, "column permutation")
    # unit affine: output row mean 0, population variance var/(var+eps)
    ones, zeros = np.ones(d, np.float32), np.zeros(d, np.float32)
    yu, _, _, _, vu = _ln(lib, xr, ones, zeros)
    yd = yu.astype(np.float64)
    assert np.all(np.abs(yd.mean(axis=1)) <= 1e-6), "unit affine: row mean != 0"
    want = vu / (vu + float(EPS32))
    np.testing.assert_allclose(yd.var(axis=1), want, rtol=2e-6)
    # in place: y written over x gives the same values
    xin = xr.copy()
    oracle.layernorm(xin, g, b, float(EPS32), lib=lib, out=xin)
    assert np.array_equal(xin, yr), "in-place LayerNorm differs"


def check_rms_invariants(lib):
    rows, d = 10, 300
    x = wl.make_x(rows, d, "normal", [18, 1])
    w = wl.make_weight(d, [18, 2])
    y0, r0, _ = _rms(lib, x, w)
    # power-of-two scale: RMS_eps(2x) == RMS_{eps/4}(x) bit for bit
    y2, _, _ = _rms(lib, (2 * x).astype(np.float32), w, EPS32)
    y3, _, _ = _rms(lib, x, w, np.float32(EPS32 / 4))
    assert np.array_equal(y2, y3), "RMS_eps(2x) != RMS_eps/4(x)"
    # the output is linear in w: w -> 2w doubles y exactly
    y4, _, _ = _rms(lib, x, (2 * w).astype(np.float32))
    assert np.array_equal(y4, 2 * y0), "RMS not linear in w"
    # y / (x w) is the per-row rstd
    ratio = y0.astype(np.float64) / (x.astype(np.float64) * w)
    np.testing.assert_allclose(ratio, np.repeat(r0[:, None].astype(np.float64), d, axis=1),
                               rtol=2e-7)
    cp = _rng([18, 3]).permutation(d)
    yc, _, _ = _rms(lib, np.ascontiguousarray(x[:, cp]), w[cp])
    _assert_ulps(yc, y0[:, cp], 1, "rms column permutation")
    xin = x.copy()
    oracle.rmsnorm(xin, w, float(EPS32), lib=lib, out=xin)
    assert np.array_equal(xin, y0), "in-place RMSNorm differs"


# ----------------------------------------------------------------------------
# residual add fused before the norm

def check_add_norm(lib):
    """h is the float32 sum bit for bit; y is the pinned definition applied to h.

    Pinned against: numpy's float32 addition (h), torch float64 LayerNorm /
    RMSNorm of that sum (y within 1 ulp), a zero residual giving the plain
    operation bit for bit, and exact brute force on a tiny case."""
    import torch
    import torch.nn.functional as F
    for rows, d in ((33, 1), (17, 127), (40, 768)):
        x = wl.make_x(rows, d, "offset", [19, rows, d])
        r = wl.make_x(rows, d, "normal", [20, rows, d])
        g, b = wl.make_affine(d, [19, d])
        w = wl.make_weight(d, [19, d])
        h32 = (x + r).astype(np.float32)               # numpy float32 add, round to nearest even
        y, h, mean, rstd = oracle.add_layernorm(x, r, g, b, float(EPS32), lib=lib)
        assert np.array_equal(h, h32), "h != x + r in float32"
        ty, tm, tr = torch.native_layer_norm(torch.from_numpy(h32).double(), (d,),
                                             torch.from_numpy(g).double(),
                                             torch.from_numpy(b).double(), float(EPS32))
        _assert_ulps(y, ty.numpy().astype(np.float32), 1, f"add+ln vs torch {rows}x{d}")
        _assert_ulps(rstd, tr.reshape(-1).numpy().astype(np.float32), 1, "add+ln rstd")
        yr, hr, rr = oracle.add_rmsnorm(x, r, w, float(EPS32), lib=lib)
        assert np.array_equal(hr, h32)
        ty = F.rms_norm(torch.from_numpy(h32).double(), (d,), torch.from_numpy(w).double(),
                        eps=float(EPS32))
        _assert_ulps(yr, ty.numpy().astype(np.float32), 1, f"add+rms vs torch {rows}x{d}")
        # a zero residual is the plain operation, bit for bit
        z = np.zeros_like(x)
        assert np.array_equal(oracle.add_layernorm(x, z, g, b, float(EPS32), lib=lib)[0],
                              oracle.layernorm(x, g, b, float(EPS32), lib=lib)[0])
        assert np.array_equal(oracle.add_rmsnorm(x, z, w, float(EPS32), lib=lib)[0],
                              oracle.rmsnorm(x, w, float(EPS32), lib=lib)[0])
    # exact brute force on a tiny case with a non-trivial residual
    x = np.array([[0.5, -1.25, 2.0, 3.5]], np.float32)
    r = np.array([[1.0, 0.25, -2.5, 0.125]], np.float32)
    g = np.array([1.5, 0.5, -1.0, 2.0], np.float32)
    b = np.array([0.1, 0.2, 0.3, 0.4], np.float32)
    y, h, _, _ = oracle.add_layernorm(x, r, g, b, float(EPS32), lib=lib)
    _, _, _, ys = _exact_ln_row((x + r)[0], g, b, EPS32)
    _assert_ulps(y[0], np.array([float(t) for t in ys], np.float32), 1, "add+ln brute force")


LN_CHECKS = (check_ln_bruteforce, check_ln_vs_torch, check_ln_closed_forms, check_ln_invariants)
RMS_CHECKS = (check_rms_bruteforce, check_rms_vs_torch, check_rms_closed_forms, check_rms_invariants)
ALL_CHECKS = LN_CHECKS + RMS_CHECKS + (check_add_norm,)


# ----------------------------------------------------------------------------
# 16-bit storage: exact widening, one round-to-nearest-even narrowing

F16, BF16 = oracle.FMT_F16, oracle.FMT_BF16


def _lib_values16(bits: np.ndarray, fmt: int) -> np.ndarray:
    """float64 values of 16-bit patterns by library casts (numpy binary16,
    torch bfloat16), independent of the oracle's decoder."""
    if fmt == F16:
        return bits.view(np.float16).astype(np.float64)
    import torch
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def _finite_table(fmt: int):
    """Every finite non-negative value of the format, ascending, with its pattern."""
    bits = np.arange(0, 0x8000, dtype=np.uint16)
    vals = _lib_values16(bits, fmt)
    keep = np.isfinite(vals)
    order = np.argsort(vals[keep], kind="stable")
    return vals[keep][order], bits[keep][order]


def _nearest16(v: Fraction | float, table, fmt: int) -> int:
    """The format's pattern nearest to the exact value v, ties to the even
    pattern, overflow past the last midpoint to infinity, the sign kept (a
    negative value too small for the format gives -0): the definition,
    evaluated by search over every finite value."""
    vals, bits = table
    f = Fraction(v)
    neg = f < 0
    a = -f if neg else f
    i = int(np.searchsorted(vals, float(a)))
    cands = {max(0, min(len(vals) - 1, j)) for j in (i - 2, i - 1, i, i + 1)}
    best = None
    for j in sorted(cands):
        dist = abs(Fraction(float(vals[j])) - a)
        key = (dist, int(bits[j]) & 1)
        if best is None or key < best[0]:
            best = (key, j)
    j = best[1]
    top = Fraction(float(vals[-1]))
    ulp_top = top - Fraction(float(vals[-2]))
    if a >= top + ulp_top / 2:                       # at or past the overflow midpoint
        out = 0x7C00 if fmt == F16 else 0x7F80
    else:
        out = int(bits[j])
    return out | 0x8000 if neg else out


def check_widen16(lib):
    """Every one of the 65536 patterns of each format decodes to the value the
    library casts give (NaN patterns to NaN)."""
    bits = np.arange(65536, dtype=np.uint16)
    for fmt in (F16, BF16):
        got = oracle.widen16(bits, fmt, lib=lib).astype(np.float64)
        want = _lib_values16(bits, fmt)
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), f"fmt {fmt}: NaN patterns"
        assert np.array_equal(got[~nan], want[~nan]), f"fmt {fmt}: decoded values"
        # signed zeros keep their sign
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def check_round16(lib):
    """Narrowing is round to nearest, ties to even, from the float64 value.

    Pinned by (a) the nearest-value search over every finite value of the
    format with exact rational distances, on random magnitudes from the
    subnormals to past overflow, (b) every midpoint between neighbours and
    the doubles just beside it, (c) numpy's float64 -> binary16 cast and
    torch's float32 -> bfloat16 cast on float32 values."""
    rng = _rng([61])
    for fmt, (lo, hi) in ((F16, (-27, 17)), (BF16, (-136, 129))):
        table = _finite_table(fmt)
        e = rng.uniform(lo, hi, 4000)
        v = np.ldexp(rng.uniform(0.5, 1.0, e.size), np.floor(e).astype(int)) * rng.choice([-1.0, 1.0], e.size)
        got = oracle.round16(v, fmt, lib=lib)
        want = np.array([_nearest16(float(t), table, fmt) for t in v], np.uint16)
        assert np.array_equal(got, want), f"fmt {fmt}: nearest value"
        # midpoints between neighbours (exact in float64), and one double ulp each side
        vals, bits = table
        idx = rng.integers(0, len(vals) - 1, 3000)
        mid = (vals[idx] + vals[idx + 1]) / 2
        even = np.where(bits[idx] % 2 == 0, bits[idx], bits[idx + 1])
        assert np.array_equal(oracle.round16(mid, fmt, lib=lib), even), f"fmt {fmt}: ties to even"
        assert np.array_equal(oracle.round16(np.nextafter(mid, -np.inf), fmt, lib=lib), bits[idx])
        assert np.array_equal(oracle.round16(np.nextafter(mid, np.inf), fmt, lib=lib), bits[idx + 1])
        assert np.array_equal(oracle.round16(-mid, fmt, lib=lib), even | 0x8000)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-30, 18, 20000))
    with np.errstate(over="ignore"):
        want16 = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.round16(x, F16, lib=lib), want16)
    import torch
    x32 = (rng.standard_normal(20000) * np.exp2(rng.integers(-140, 120, 20000))).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round16(x32.astype(np.float64), BF16, lib=lib), want)


def check_add16(lib):
    """h = x + r rounded once: the nearest-value search on the exact rational
    sum, including exponent gaps past float64's precision (bfloat16)."""
    rng = _rng([62])
    for fmt in (F16, BF16):
        table = _finite_table(fmt)
        vals, bits = table
        n = 3000
        xi = rng.integers(0, len(vals), n)
        ri = rng.integers(0, len(vals), n)
        xb = bits[xi] | np.where(rng.random(n) < 0.5, 0x8000, 0).astype(np.uint16)
        rb = bits[ri] | np.where(rng.random(n) < 0.5, 0x8000, 0).astype(np.uint16)
        # and close pairs, where cancellation and ties are likely
        xb[:500] = bits[rng.integers(len(vals) // 2, len(vals) - 1, 500)]
        rb[:500] = (xb[:500] + rng.integers(-3, 4, 500).astype(np.uint16)) | 0x8000
        got = oracle.add16(xb, rb, fmt, lib=lib)
        xv, rv = _lib_values16(xb, fmt), _lib_values16(rb, fmt)
        for k in range(n):
            s = Fraction(float(xv[k])) + Fraction(float(rv[k]))
            w = _nearest16(s, table, fmt)
            if s == 0:
                assert got[k] & 0x7FFF == 0, f"fmt {fmt}: zero sum"
            else:
                assert int(got[k]) == w, f"fmt {fmt}: {xv[k]!r} + {rv[k]!r}"


def check_norm16(lib):
    """LayerNorm / RMSNorm over 16-bit storage: the outputs are torch's
    float64 routines on the exactly widened inputs, rounded once (bit for bit
    away from rounding midpoints); a zero row gives the rounded bias."""
    import torch
    import torch.nn.functional as F
    for fmt in (F16, BF16):
        for rows, d, pat in ((16, 768, "offset"), (9, 33, "normal"), (4, 1, "normal")):
            x16 = wl.make_x16(rows, d, pat, [63, rows, d], fmt)
            g, b = wl.make_affine(d, [63, d])
            w = wl.make_weight(d, [63, d])
            xd = torch.from_numpy(_lib_values16(x16, fmt).reshape(rows, d))
            y, y64, mean, rstd = oracle.layernorm16(x16, fmt, g, b, float(EPS32), lib=lib)
            ty, tm, tr = torch.native_layer_norm(xd, (d,), torch.from_numpy(g).double(),
                                                 torch.from_numpy(b).double(), float(EPS32))
            assert np.allclose(y64, ty.numpy(), rtol=1e-12, atol=1e-12), "y64 vs torch"
            table = _finite_table(fmt)
            wantb = np.array([_nearest16(float(t), table, fmt) for t in ty.numpy().ravel()])
            agree = np.mean(y.ravel() == wantb)
            assert agree >= 0.999, f"fmt {fmt}: only {agree:.4f} of outputs round as torch's"
            _assert_ulps(mean, tm.reshape(-1).numpy().astype(np.float32), 1, "mean16")
            _assert_ulps(rstd, tr.reshape(-1).numpy().astype(np.float32), 1, "rstd16")
            yr, yr64, rr = oracle.rmsnorm16(x16, fmt, w, float(EPS32), lib=lib)
            tyr = F.rms_norm(xd, (d,), torch.from_numpy(w).double(), eps=float(EPS32)).numpy()
            assert np.allclose(yr64, tyr, rtol=1e-12, atol=1e-12), "rms y64 vs torch"
        # zero rows: y is beta rounded once to the format (a library cast of float32)
        d = 40
        g, b = wl.make_affine(d, [64, d])
        z = np.zeros((3, d), np.uint16)
        y, _, mean, _ = oracle.layernorm16(z, fmt, g, b, float(EPS32), lib=lib)
        assert np.array_equal(y, np.broadcast_to(wl.quantize16(b, fmt), y.shape)), "zero rows give beta"
        assert not np.any(mean)
        # fused: h is the stored sum and y the norm of that stored h
        x16 = wl.make_x16(5, 96, "offset", [65], fmt)
        r16 = wl.make_x16(5, 96, "normal", [66], fmt)
        g, b = wl.make_affine(96, [65])
        y, y64, h, mean, rstd = oracle.add_layernorm16(x16, r16, fmt, g, b, float(EPS32), lib=lib)
        assert np.array_equal(h, oracle.add16(x16, r16, fmt, lib=lib))
        y2, y642, _, _ = oracle.layernorm16(h, fmt, g, b, float(EPS32), lib=lib)
        assert np.array_equal(y, y2) and np.array_equal(y64, y642)


def check_tolerance16(lib):
    """The 16-bit acceptance bound: a float32-accurate value rounded to
    nearest passes; two ulps off fails; NaN fails."""
    rng = _rng([67])
    for fmt in (F16, BF16):
        ref = rng.standard_normal(5000) * 2.0
        tau = 1e-5 + 1e-4 * np.abs(ref)
        near = oracle.round16(ref + 0.99 * tau * rng.choice([-1, 1], ref.size), fmt, lib=lib)
        assert oracle.tolerance_ok16(near, ref, fmt, lib=lib)[0]
        step = oracle.round16(ref, fmt, lib=lib).astype(np.int64)
        off = np.where(step & 0x8000, step - 2, step + 2).astype(np.uint16)   # two ulps toward zero
        big = np.abs(ref) > 0.01
        ok, _, _ = oracle.tolerance_ok16(off[big], ref[big], fmt, lib=lib)
        assert not ok
        nanb = np.array([0x7E00 if fmt == F16 else 0x7FC0], np.uint16)
        assert not oracle.tolerance_ok16(nanb, np.array([0.0]), fmt, lib=lib)[0]


STORAGE16_CHECKS = (check_widen16, check_round16, check_add16, check_norm16, check_tolerance16)
ALL_CHECKS = ALL_CHECKS + STORAGE16_CHECKS


# ----------------------------------------------------------------------------
# backward: the exact derivative of the pinned forward definitions

def _exact_stats(x, eps):
    """float64 mean and rstd of each row, from the forward oracle's float64
    statistics (mean64, var64)."""
    _, _, _, m64, v64 = oracle.layernorm(x, np.ones(x.shape[1], np.float32),
                                         np.zeros(x.shape[1], np.float32), float(eps))
    return m64, 1.0 / np.sqrt(v64 + float(np.float32(eps)))


def check_bwd_autograd(lib):
    """dx, dgamma, dbeta (and RMSNorm dx, dw) equal torch's float64 autograd
    through F.layer_norm / F.rms_norm when the exact statistics are passed."""
    import torch
    import torch.nn.functional as F
    for rows, d, pat in ((7, 33, "offset"), (5, 1, "normal"), (9, 256, "normal"), (4, 129, "tiny")):
        x = wl.make_x(rows, d, pat, [70, rows, d])
        dy = wl.make_x(rows, d, "normal", [71, rows, d])
        g, b = wl.make_affine(d, [70, d])
        w = wl.make_weight(d, [70, d])
        m64, r64 = _exact_stats(x, EPS32)
        out = oracle.layernorm_bwd(dy, x, g, m64, r64, lib=lib)
        xt = torch.from_numpy(x).double().requires_grad_(True)
        gt = torch.from_numpy(g).double().requires_grad_(True)
        bt = torch.from_numpy(b).double().requires_grad_(True)
        y = F.layer_norm(xt, (d,), gt, bt, float(EPS32))
        y.backward(torch.from_numpy(dy).double())
        for got, want, what in ((out["dx64"], xt.grad, "dx"), (out["dgamma64"], gt.grad, "dgamma"),
                                (out["dbeta64"], bt.grad, "dbeta")):
            want = want.numpy()
            scale = np.abs(want).max() + 1.0       # gradients here are O(1); d = 1 gives dgamma = 0
            assert np.abs(got - want).max() <= 1e-11 * scale, f"LN {what} {rows}x{d} {pat}"
        r64 = 1.0 / np.sqrt((x.astype(np.float64) ** 2).mean(axis=1) + float(EPS32))
        o2 = oracle.rmsnorm_bwd(dy, x, w, r64, lib=lib)
        xt = torch.from_numpy(x).double().requires_grad_(True)
        wt = torch.from_numpy(w).double().requires_grad_(True)
        F.rms_norm(xt, (d,), wt, eps=float(EPS32)).backward(torch.from_numpy(dy).double())
        for got, want, what in ((o2["dx64"], xt.grad, "dx"), (o2["dw64"], wt.grad, "dw")):
            want = want.numpy()
            scale = np.abs(want).max() + 1.0
            assert np.abs(got - want).max() <= 1e-11 * scale, f"RMS {what} {rows}x{d} {pat}"


def check_bwd_finite_differences(lib):
    """Central differences of the float64 forward outputs (y64 of the pinned
    forward oracle) match the backward, on dyadic inputs where x +- h and
    gamma +- h are exact in float32 (no torch involved)."""
    rng = _rng([72])
    rows, d, h = 3, 6, 2.0 ** -12
    x = (rng.integers(-2048, 2048, (rows, d)) * 2.0 ** -10).astype(np.float32)
    dy = (rng.integers(-64, 64, (rows, d)) * 2.0 ** -5).astype(np.float32)
    g = (1 + rng.integers(-64, 64, d) * 2.0 ** -8).astype(np.float32)
    b = (rng.integers(-64, 64, d) * 2.0 ** -8).astype(np.float32)

    def loss_ln(xv, gv, bv):
        y64 = np.empty(xv.shape)
        oracle.layernorm(xv, gv, bv, float(EPS32), lib=lib, y64=y64)
        return float((y64 * dy).sum())

    def loss_rms(xv, wv):
        y64 = np.empty(xv.shape)
        oracle.rmsnorm(xv, wv, float(EPS32), lib=lib, y64=y64)
        return float((y64 * dy).sum())

    m64, r64 = _exact_stats(x, EPS32)
    out = oracle.layernorm_bwd(dy, x, g, m64, r64, lib=lib)
    rr = 1.0 / np.sqrt((x.astype(np.float64) ** 2).mean(axis=1) + float(EPS32))
    o2 = oracle.rmsnorm_bwd(dy, x, g, rr, lib=lib)
    for i in range(rows):
        for j in range(d):
            xp, xm = x.copy(), x.copy()
            xp[i, j] += np.float32(h)
            xm[i, j] -= np.float32(h)
            fd = (loss_ln(xp, g, b) - loss_ln(xm, g, b)) / (2 * h)
            assert abs(fd - out["dx64"][i, j]) <= 1e-5 * (1 + abs(fd)), ("LN dx", i, j, fd, out["dx64"][i, j])
            fd = (loss_rms(xp, g) - loss_rms(xm, g)) / (2 * h)
            assert abs(fd - o2["dx64"][i, j]) <= 1e-5 * (1 + abs(fd)), ("RMS dx", i, j)
    for j in range(d):
        gp, gm = g.copy(), g.copy()
        gp[j] += np.float32(h)
        gm[j] -= np.float32(h)
        fd = (loss_ln(x, gp, b) - loss_ln(x, gm, b)) / (2 * h)
        assert abs(fd - out["dgamma64"][j]) <= 1e-6 * (1 + abs(fd)), ("dgamma", j)
        fd = (loss_rms(x, gp) - loss_rms(x, gm)) / (2 * h)
        assert abs(fd - o2["dw64"][j]) <= 1e-6 * (1 + abs(fd)), ("dw", j)
        bp, bm = b.copy(), b.copy()
        bp[j] += np.float32(h)
        bm[j] -= np.float32(h)
        fd = (loss_ln(x, g, bp) - loss_ln(x, g, bm)) / (2 * h)
        assert abs(fd - out["dbeta64"][j]) <= 1e-6 * (1 + abs(fd)), ("dbeta", j)


def check_bwd_invariants(lib):
    """Shift invariance of LayerNorm makes every dx row sum to zero; at eps = 0
    scale invariance makes dx orthogonal to (x - mu) (LayerNorm) and to x
    (RMSNorm); a power-of-two scale of dy scales every gradient exactly."""
    for rows, d in ((6, 40), (3, 999)):
        x = wl.make_x(rows, d, "offset", [73, d])
        dy = wl.make_x(rows, d, "normal", [74, d])
        g, _ = wl.make_affine(d, [73, d])
        m64, r64 = _exact_stats(x, EPS32)
        out = oracle.layernorm_bwd(dy, x, g, m64, r64, lib=lib)
        scale = np.abs(out["dx64"]).sum(axis=1)
        assert np.all(np.abs(out["dx64"].sum(axis=1)) <= 1e-12 * scale), "LN dx rows do not sum to 0"
        m0, r0 = _exact_stats(x, 0.0)
        o0 = oracle.layernorm_bwd(dy, x, g, m0, r0, lib=lib)
        c = x.astype(np.float64) - m0[:, None]
        dot = (o0["dx64"] * c).sum(axis=1)
        assert np.all(np.abs(dot) <= 1e-11 * (np.abs(o0["dx64"] * c).sum(axis=1))), "LN eps=0 scale"
        rr0 = 1.0 / np.sqrt((x.astype(np.float64) ** 2).mean(axis=1))
        o2 = oracle.rmsnorm_bwd(dy, x, g, rr0, lib=lib)
        dot = (o2["dx64"] * x).sum(axis=1)
        assert np.all(np.abs(dot) <= 1e-11 * np.abs(o2["dx64"] * x).sum(axis=1)), "RMS eps=0 scale"
        o4 = oracle.layernorm_bwd((dy * np.float32(4)).astype(np.float32), x, g, m64, r64, lib=lib)
        for k in ("dx64", "dgamma64", "dbeta64"):
            assert np.array_equal(o4[k], 4 * out[k]), f"dy scale {k}"


def check_bwd16(lib):
    """16-bit backward: the float32 backward on the exactly widened inputs with
    dx rounded once; and the column-sum acceptance bound passes a sum whose
    terms carry float32 rounding and refuses one missing row."""
    for fmt in (F16, BF16):
        rows, d = 12, 96
        x16 = wl.make_x16(rows, d, "offset", [75], fmt)
        dy16 = wl.make_x16(rows, d, "normal", [76], fmt)
        g, _ = wl.make_affine(d, [75])
        xw = oracle.widen16(x16, fmt, lib=lib)
        m64, r64 = _exact_stats(xw, EPS32)
        o16 = oracle.layernorm_bwd16(dy16, x16, fmt, g, m64, r64, lib=lib)
        o32 = oracle.layernorm_bwd(oracle.widen16(dy16, fmt, lib=lib), xw, g, m64, r64, lib=lib)
        assert np.array_equal(o16["dx64"], o32["dx64"])
        assert np.array_equal(o16["dx16"], oracle.round16(o32["dx64"], fmt, lib=lib))
    # the column-sum bound
    rows, d = 4096, 64
    x = wl.make_x(rows, d, "normal", [77])
    dy = wl.make_x(rows, d, "normal", [78])
    g, _ = wl.make_affine(d, [77])
    m64, r64 = _exact_stats(x, EPS32)
    o = oracle.layernorm_bwd(dy, x, g, m64, r64, lib=lib)
    xh32 = ((x - m64[:, None].astype(np.float32)) * r64[:, None].astype(np.float32)).astype(np.float32)
    terms32 = (dy * xh32).astype(np.float32)
    got = terms32.astype(np.float64).sum(axis=0).astype(np.float32)
    assert oracle.colsum_tolerance_ok(got, o["dgamma64"], o["abs_dgamma"])[0]
    # any split of the rows into partial sums and each of those again,
    # every partial rounded once to float32, and any order of the float64
    # additions
    rng = np.random.default_rng(79)

    def split_sum(idx, levels):
        if levels == 0 or len(idx) < 2:
            return terms32[idx].astype(np.float64).sum(axis=0).astype(np.float32)
        parts = int(rng.integers(2, min(len(idx), 64) + 1))
        cut = np.sort(rng.choice(np.arange(1, len(idx)), parts - 1, replace=False))
        partial = [split_sum(idx[i:j], levels - 1) for i, j in zip(np.r_[0, cut], np.r_[cut, len(idx)])]
        return np.sum(np.asarray(partial, np.float64)[rng.permutation(parts)], axis=0).astype(np.float32)

    for levels in (1, 2, 3):
        split = split_sum(rng.permutation(rows), levels)
        assert oracle.colsum_tolerance_ok(split, o["dgamma64"], o["abs_dgamma"])[0], levels
    missing = terms32[1:].astype(np.float64).sum(axis=0).astype(np.float32)
    assert not oracle.colsum_tolerance_ok(missing, o["dgamma64"], o["abs_dgamma"])[0]


BWD_CHECKS = (check_bwd_autograd, check_bwd_finite_differences, check_bwd_invariants, check_bwd16)
ALL_CHECKS = ALL_CHECKS + BWD_CHECKS


def check_dx_tolerance(lib):
    """The dx acceptance bound passes an evaluation of the same formula with
    every term and product in float32, a row's terms added in float32 in
    groups of eight consecutive ones and in float64 from there, in either
    order, each mean rounded once (including rows of zero variance, where
    rstd ~ 1/sqrt(eps) amplifies the rounding), and refuses dx without the
    mean of g or with a flipped projection term."""
    for rows, d, pat in ((64, 1, "normal"), (32, 256, "normal"), (16, 8, "zero"), (16, 77, "offset")):
        x = wl.make_x(rows, d, pat, [80, d])
        dy = wl.make_x(rows, d, "normal", [81, d])
        g, _ = wl.make_affine(d, [80, d])
        _, mean, rstd, _, _ = oracle.layernorm(x, g, np.zeros(d, np.float32), float(EPS32), lib=lib)
        ref = oracle.layernorm_bwd(dy, x, g, mean, rstd, lib=lib)
        # every term and product rounded to float32; a row's terms summed
        # pairwise in float32 in groups of eight, the group sums in float64
        # (forwards, then backwards); each mean rounded once
        f = np.float32
        xh = ((x - mean[:, None]).astype(f) * rstd[:, None]).astype(f)
        gg = (dy * g).astype(f)
        gx = (gg * xh).astype(f)

        def groups8(t):
            pad = np.zeros((rows, -(-d // 8) * 8), f)
            pad[:, :d] = t
            v = pad.reshape(rows, -1, 8)
            while v.shape[2] > 1:
                v = (v[:, :, 0::2] + v[:, :, 1::2]).astype(f)
            return v[:, :, 0].astype(np.float64)

        for order in (slice(None), slice(None, None, -1)):
            m1 = (np.cumsum(groups8(gg)[:, order], axis=1)[:, -1] / d).astype(f)
            m2 = (np.cumsum(groups8(gx)[:, order], axis=1)[:, -1] / d).astype(f)
            dx32 = (rstd[:, None] * ((gg - m1[:, None]).astype(f) - (xh * m2[:, None]).astype(f)).astype(f)).astype(f)
            ok, _, ratio = oracle.dx_tolerance_ok(dx32, ref["dx64"], ref["dx_scale"])
            assert ok, f"float32 evaluation refused ({rows}x{d} {pat}, ratio {ratio:.2f})"
        if d > 1 and pat != "zero":
            bad = ref["dx64"] + rstd[:, None].astype(np.float64) * (gg.astype(np.float64).mean(axis=1))[:, None]
            assert not oracle.dx_tolerance_ok(bad, ref["dx64"], ref["dx_scale"])[0], "mean of g dropped"
            proj = 2 * (rstd[:, None] * xh.astype(np.float64) * m2[:, None])   # the term with its sign flipped
            assert not oracle.dx_tolerance_ok(ref["dx64"] + proj, ref["dx64"], ref["dx_scale"])[0], "projection sign"


BWD_CHECKS = BWD_CHECKS + (check_dx_tolerance,)
ALL_CHECKS = ALL_CHECKS + (check_dx_tolerance,)
