"""Negative controls: the checks must fail when the definition is broken.

Each case rebuilds the C oracle with one planted mistake (ORACLE_PLANT) in a
temporary directory and requires the pin suite to reject it.  The first two
are the controls of "RMSNorm on an RTX 5070" (section "Correctness before
timing"): without epsilon the zero input gives NaN, and a dropped final
column leaves a sentinel in the output.  Everything runs on the CPU.
"""
import numpy as np
import pytest

import oracle
import oracle_pins as pins
from oracle import build as obuild
from row_wise_normalization_layernorm_amd import workloads as wl

PLANTS = {
    1: ("layernorm eps removed", pins.LN_CHECKS),
    2: ("layernorm final column dropped", pins.LN_CHECKS),
    3: ("layernorm unbiased variance", pins.LN_CHECKS),
    4: ("layernorm bias dropped", pins.LN_CHECKS),
    5: ("layernorm scale indexed by row", pins.LN_CHECKS),
    6: ("layernorm deviation sign flipped", pins.LN_CHECKS),
    7: ("rmsnorm eps removed", pins.RMS_CHECKS),
    8: ("rmsnorm wrong denominator", pins.RMS_CHECKS),
    9: ("layernorm eps outside the root", pins.LN_CHECKS),
    10: ("add+layernorm residual dropped", (pins.check_add_norm,)),
    11: ("add+rmsnorm input dropped", (pins.check_add_norm,)),
    12: ("16-bit narrowing truncates", (pins.check_round16, pins.check_norm16, pins.check_tolerance16)),
    13: ("16-bit narrowing ties away from zero", (pins.check_round16, pins.check_add16)),
    14: ("16-bit residual dropped", (pins.check_add16, pins.check_norm16)),
    15: ("layernorm backward mean of g dropped", pins.BWD_CHECKS),
    16: ("layernorm backward projection sign", pins.BWD_CHECKS),
    17: ("layernorm backward dgamma without the mean", pins.BWD_CHECKS),
    18: ("rmsnorm backward outer rstd dropped", pins.BWD_CHECKS),
}


@pytest.fixture(scope="module")
def planted(tmp_path_factory):
    d = tmp_path_factory.mktemp("planted")
    libs = {}
    for k in PLANTS:
        path = str(d / f"liboracle_plant{k}.so")
        obuild.build(path, plant=k)
        libs[k] = oracle.load(path)
        assert libs[k].oracle_plant() == k
    return libs


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda k: PLANTS[k][0].replace(" ", "_"))
def test_planted_mistake_is_caught(planted, plant):
    lib = planted[plant]
    caught = []
    for check in PLANTS[plant][1]:
        try:
            check(lib)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"no pin caught the planted mistake: {PLANTS[plant][0]}"


def test_no_epsilon_gives_nan_on_zero_input(planted):
    d = 64
    g, b = wl.make_affine(d, 0)
    x = np.zeros((8, d), np.float32)
    good = oracle.layernorm(x, g, b, wl.EPS)[0]
    bad = oracle.layernorm(x, g, b, wl.EPS, lib=planted[1])[0]
    assert not np.all(np.isfinite(bad))
    assert not oracle.tolerance_ok(bad, good)[0]
    badr = oracle.rmsnorm(x, wl.make_weight(d, 0), wl.EPS, lib=planted[7])[0]
    assert not oracle.tolerance_ok(badr, np.zeros_like(x))[0]


def test_dropped_final_column_leaves_sentinel(planted):
    x = wl.make_x(16, 33, "normal", 5)
    g, b = wl.make_affine(33, 5)
    sentinel = np.float32(-7777.0)
    out = np.full_like(x, sentinel)
    oracle.layernorm(x, g, b, wl.EPS, lib=planted[2], out=out)
    assert np.all(out[:, -1] == sentinel)
    good = oracle.layernorm(x, g, b, wl.EPS)[0]
    assert not oracle.tolerance_ok(out, good)[0]
