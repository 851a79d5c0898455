"""The shipped CPU oracle against exact brute force, torch's float64 routines,
closed forms and invariants (the checks live in oracle_pins.py)."""
import json
import os

import numpy as np
import pytest

import oracle
import oracle_pins as pins
from row_wise_normalization_layernorm_amd import workloads as wl


@pytest.fixture(scope="module")
def lib():
    lib = oracle.load()
    assert lib.oracle_plant() == 0, "the shipped oracle must carry no planted mistake"
    return lib


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(lib, check):
    check(lib)


def test_protocol_fixture_matches_generators():
    """The pages' protocol constants drive the inputs and the acceptance bound."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "protocol.json")) as f:
        proto = json.load(f)
    assert proto["eps"] == wl.EPS
    assert proto["cases"] == len(proto["widths"]) * len(proto["patterns"]) * proto["layouts"]
    for p in proto["patterns"]:
        assert p in wl.PATTERNS
    # the acceptance helper implements exactly the stated bound
    ref = np.array([0.0, 1.0, -100.0])
    bound = proto["atol"] + proto["rtol"] * np.abs(ref)
    assert oracle.tolerance_ok(ref + 0.999 * bound, ref)[0]
    assert not oracle.tolerance_ok(ref + 1.001 * bound, ref)[0]
    assert not oracle.tolerance_ok(np.array([np.nan, 1.0, -100.0]), ref)[0]


def test_generators_are_seeded_and_shaped():
    a = wl.make_x(7, 33, "normal", [1, 2, 3])
    b = wl.make_x(7, 33, "normal", [1, 2, 3])
    assert a.dtype == np.float32 and a.flags.c_contiguous and a.shape == (7, 33)
    assert np.array_equal(a, b)
    alt = wl.make_x(2, 3, "alternating")
    assert alt.tolist() == [[1, -1, 1], [-1, 1, -1]]
    assert not np.any(wl.make_x(3, 5, "zero"))
    tiny = wl.make_x(64, 64, "tiny", 0)
    assert 1e-7 < float(np.abs(tiny).mean()) < 1e-5
    off = wl.make_x(256, 256, "offset", 0).astype(np.float64)
    assert abs(off.mean() - 0.5) < 0.05 and abs(off.std() - 3.0) < 0.05


def test_oracle_threads_are_reported():
    assert oracle.max_threads() >= 1
