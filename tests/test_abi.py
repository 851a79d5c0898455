"""The C ABI on the CPU: the library loads, exports what the header declares,
rejects bad arguments before touching a device, and its dispatcher picks an
eligible variant for every width and layout.  No kernel is launched here."""
import ctypes
import math
import os
import subprocess

import pytest

import row_wise_normalization_layernorm_amd as mn
from row_wise_normalization_layernorm_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# fake, well-aligned device addresses: validation never dereferences them
X, Y, G, BETA = 0x7F0000000000, 0x7F0100000000, 0x7F0200000000, 0x7F0300000000


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return mn.lib()


def test_exports_every_declared_symbol(L):
    declared = B.header_functions()
    assert {"mi_layernorm_fwd", "mi_rmsnorm_fwd", "mi_norm_status_string"} <= set(declared)
    for name in declared:
        assert hasattr(L, name), f"{name} declared in mi_norm.h but not exported"
    nm = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True,
                        check=True).stdout
    exported = {l.split()[-1] for l in nm.splitlines() if " T " in l and l.split()[-1].startswith("mi_")}
    assert exported == set(declared), exported ^ set(declared)


def test_header_compiles_as_plain_c():
    r = subprocess.run(["gcc", "-std=c99", "-fsyntax-only", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I/opt/rocm/include", "-x", "c", os.path.join(ROOT, "include", "mi_norm.h")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_single_hip_runtime_is_mapped(L):
    maps = {l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l}
    assert len(maps) == 1, maps


def test_status_strings(L):
    assert mn.mi_norm_status_string(0) == "MI_NORM_OK"
    assert "INVALID" in mn.mi_norm_status_string(1)
    assert "HIP" in mn.mi_norm_status_string(2)
    assert "UNKNOWN" in mn.mi_norm_status_string(7)
    assert "gfx950" in mn.mi_norm_version()


@pytest.mark.parametrize("args", [
    (0, G, BETA, Y, 4, 8, 1e-5, None, None, None),          # null x
    (X, 0, BETA, Y, 4, 8, 1e-5, None, None, None),          # null gamma
    (X, G, 0, Y, 4, 8, 1e-5, None, None, None),             # null beta
    (X, G, BETA, 0, 4, 8, 1e-5, None, None, None),          # null y
    (X, G, BETA, Y, -1, 8, 1e-5, None, None, None),         # rows < 0
    (X, G, BETA, Y, 4, 0, 1e-5, None, None, None),          # d < 1
    (X, G, BETA, Y, 4, 2**31, 1e-5, None, None, None),      # d too wide
    (X, G, BETA, Y, 4, 8, -1e-5, None, None, None),         # eps < 0
    (X, G, BETA, Y, 4, 8, math.nan, None, None, None),      # eps NaN
    (X + 2, G, BETA, Y, 4, 8, 1e-5, None, None, None),      # x not 4-byte aligned
    (X, G + 1, BETA, Y, 4, 8, 1e-5, None, None, None),      # gamma not 4-byte aligned
    (X, G, BETA, Y, 4, 8, 1e-5, 0x1001, None, None),        # mean not 4-byte aligned
    (X, G, BETA, X + 16, 4, 8, 1e-5, None, None, None),     # y partially overlaps x
    (X, G, BETA, Y, 2**62, 8, 1e-5, None, None, None),      # size overflow
    (X, Y + 64, BETA, Y, 4, 8, 1e-5, None, None, None),     # gamma inside y
    (X, G, Y, Y, 4, 8, 1e-5, None, None, None),             # beta inside y
])
def test_layernorm_rejects_bad_arguments(L, args):
    assert L.mi_layernorm_fwd(*args) == mn.MI_NORM_ERR_INVALID


@pytest.mark.parametrize("args", [
    (0, G, Y, 4, 8, 1e-5, None, None),
    (X, 0, Y, 4, 8, 1e-5, None, None),
    (X, G, 0, 4, 8, 1e-5, None, None),
    (X, G, Y, -3, 8, 1e-5, None, None),
    (X, G, Y, 4, -8, 1e-5, None, None),
    (X, G, Y, 4, 8, math.nan, None, None),
    (X, G, X + 4, 4, 8, 1e-5, None, None),
])
def test_rmsnorm_rejects_bad_arguments(L, args):
    assert L.mi_rmsnorm_fwd(*args) == mn.MI_NORM_ERR_INVALID


def test_zero_rows_is_a_no_op(L):
    # nothing is launched, so this succeeds without a device
    assert L.mi_layernorm_fwd(X, G, BETA, Y, 0, 768, 1e-5, None, None, None) == mn.MI_NORM_OK
    assert L.mi_rmsnorm_fwd(X, G, Y, 0, 8193, 1e-5, None, None) == mn.MI_NORM_OK
    assert L.mi_layernorm_fwd(X, G, BETA, X, 0, 5, 0.0, None, None, None) == mn.MI_NORM_OK
    assert L.mi_copy_f32(X, Y, 0, None) == mn.MI_NORM_OK


def test_copy_rejects_bad_arguments(L):
    assert L.mi_copy_f32(X, Y, -1, None) == mn.MI_NORM_ERR_INVALID
    assert L.mi_copy_f32(0, Y, 4, None) == mn.MI_NORM_ERR_INVALID
    assert L.mi_copy_f32(X, X + 8, 16, None) == mn.MI_NORM_ERR_INVALID
    assert L.mi_copy_f32(X, X, 16, None) == mn.MI_NORM_ERR_INVALID


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        mn.mi_layernorm_fwd(x, torch.ones(8), torch.zeros(8), x, 4, 8)


def test_binding_raises_status(L):
    with pytest.raises(mn.MiNormError) as e:
        mn.mi_layernorm_fwd(X, G, BETA, Y, 4, 0)
    assert e.value.status == mn.MI_NORM_ERR_INVALID


# --- variant table and dispatch (host logic) ---------------------------------

def _infos():
    return [(i, mn.mi_norm_variant_name(i), mn.mi_norm_variant_get_info(i))
            for i in range(mn.mi_norm_variant_count())]


def test_select_rejects_negative_rows(L):
    assert mn.mi_norm_select_variant(0, -1, 768, X, Y, G, BETA) == -1


def test_variant_table_is_consistent(L):
    infos = _infos()
    names = [n for _, n, _ in infos]
    assert len(set(names)) == len(names)
    assert mn.mi_norm_variant_name(len(infos)) is None
    assert mn.mi_norm_variant_name(-1) is None
    for i, n, v in infos:
        assert n.startswith("ln_" if v["op"] == mn.OP_LAYERNORM else "rms_")
        if v["looped"]:
            assert v["max_d"] == 2**63 - 1 and v["rows_per_block"] == 1
            continue
        assert v["max_d"] == v["vec"] * v["lanes_per_row"] * v["waves_per_row"] * v["slots"]
        if v["waves_per_row"] == 1:
            assert v["rows_per_block"] == v["waves_per_block"] * 64 // v["lanes_per_row"]
        else:
            assert v["lanes_per_row"] == 64
            assert v["rows_per_block"] * v["waves_per_row"] == v["waves_per_block"]
        assert v["waves_per_block"] * 64 <= 1024
        assert v["needs_aligned"] == (1 if v["vec"] == 4 and not v["peel"] else 0)
    ops = {v["op"] for _, _, v in infos}
    assert ops == {mn.OP_LAYERNORM, mn.OP_RMSNORM}


WIDTHS = sorted({1, 2, 3, 4, 5, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 255, 256,
                 257, 511, 512, 513, 767, 768, 769, 1000, 1023, 1024, 1025, 2047, 2048, 2049, 3000,
                 3072, 4095, 4096, 4097, 6144, 8191, 8192, 8193, 12288, 16383, 16384, 16385, 32767,
                 32768, 32769, 65536, 100003, 2**20})


@pytest.mark.parametrize("op", [mn.OP_LAYERNORM, mn.OP_RMSNORM])
@pytest.mark.parametrize("layout", ["aligned", "x_y_same_phase", "x_y_different_phase"])
def test_dispatch_picks_an_eligible_covering_variant(L, op, layout):
    if layout == "aligned":
        x, y = X, Y
    elif layout == "x_y_same_phase":
        x, y = X + 4, Y + 4
    else:
        x, y = X + 4, Y + 8
    p1 = BETA if op == mn.OP_LAYERNORM else None
    for d in WIDTHS:
        vid = mn.mi_norm_select_variant(op, 4096, d, x, y, G, p1)
        assert vid >= 0, (op, d, layout)
        v = mn.mi_norm_variant_get_info(vid)
        assert v["op"] == op
        assert mn.mi_norm_variant_eligible(vid, op, d, x, y, G, p1), (d, layout, mn.mi_norm_variant_name(vid))
        assert v["looped"] or v["max_d"] >= d
        if layout == "aligned" and d % 4 == 0:
            assert v["vec"] == 4 and not v["peel"], (d, mn.mi_norm_variant_name(vid))
        if layout == "x_y_different_phase":
            assert v["vec"] == 1, (d, mn.mi_norm_variant_name(vid))
        if layout == "aligned" and d % 4 and 256 <= d <= 32768:
            assert v["peel"], (d, mn.mi_norm_variant_name(vid))


def test_dispatch_examples(L):
    sel = lambda op, d, rows=4096, x=X, y=Y: mn.mi_norm_variant_name(
        mn.mi_norm_select_variant(op, rows, d, x, y, G, BETA if op == 0 else None))
    assert sel(0, 768) == "ln_4_p0_l64_w1_q3_b16"            # 256 workgroups of 16 rows
    assert sel(0, 768, rows=1000) == "ln_4_p0_l64_w2_q2_b4"  # few rows: two waves per row
    assert sel(0, 2048, rows=1024) == "ln_4_p0_l64_w4_q2_b4"
    assert sel(0, 4096, rows=4096) == "ln_4_p0_l64_w4_q4_b16"
    assert sel(0, 8192, rows=32768) == "ln_4_p0_l64_w8_q4_b16"
    assert sel(0, 128, rows=512) == "ln_4_p0_l32_w1_q1_b4"
    assert sel(1, 8193, rows=256) == "rms_4_p1_l64_w16_q3_b16"
    assert sel(0, 1, rows=64) == "ln_1_p0_l16_w1_q1_b4"
    assert "_loop_" in sel(0, 2**20)
    # gamma misaligned only: no 128-bit parameter reads, so not the aligned path
    assert mn.mi_norm_variant_get_info(mn.mi_norm_select_variant(0, 4096, 768, X, Y, G + 4, BETA))["needs_aligned"] == 0


def test_workgroup_size_follows_row_count(L):
    for d in (768, 2048, 4096, 8192, 16384):
        for rows in (1, 100, 1000, 5000, 100000):
            v = mn.mi_norm_variant_get_info(mn.mi_norm_select_variant(0, rows, d, X, Y, G, BETA))
            need = 512 if v["waves_per_row"] > 1 else 256
            per16 = 16 // v["waves_per_row"]
            if v["waves_per_block"] < 16:
                # a 16-wave workgroup would have left too few workgroups
                assert -(-rows // per16) < need, (d, rows)
            else:
                assert -(-rows // v["rows_per_block"]) >= need or v["waves_per_row"] == 16, (d, rows)


def test_rows_spread_over_more_waves_when_few(L):
    # about four accesses per lane with many rows; more waves per row with few
    for d, rows, wpr, q in ((768, 4096, 1, 3), (2048, 4096, 2, 4), (2048, 1024, 4, 2),
                            (4096, 4096, 4, 4), (8192, 32768, 8, 4), (16384, 8192, 16, 4),
                            (768, 100, 2, 2), (32768, 64, 16, 8)):
        v = mn.mi_norm_variant_get_info(mn.mi_norm_select_variant(0, rows, d, X, Y, G, BETA))
        assert (v["waves_per_row"], v["slots"]) == (wpr, q), (d, rows, v)


def test_eligibility_rules(L):
    infos = _infos()
    for i, n, v in infos:
        op = v["op"]
        p1 = BETA if op == 0 else None
        # the other operation never fits
        assert not mn.mi_norm_variant_eligible(i, 1 - op, 64, X, Y, G, BETA)
        if v["needs_aligned"]:
            assert not mn.mi_norm_variant_eligible(i, op, 64, X + 4, Y, G, p1)
            assert not mn.mi_norm_variant_eligible(i, op, 6, X, Y, G, p1)
        if not v["looped"]:
            assert not mn.mi_norm_variant_eligible(i, op, v["max_d"] + 4, X, Y, G, p1)
    assert not mn.mi_norm_variant_eligible(-1, 0, 8, X, Y, G, BETA)
    assert L.mi_layernorm_fwd_variant(10**6, X, G, BETA, Y, 4, 8, 1e-5, None, None, None) == mn.MI_NORM_ERR_INVALID
