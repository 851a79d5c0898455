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


# --- fused residual add: validation and aliasing ------------------------------

R_, H_ = 0x7F0400000000, 0x7F0500000000


@pytest.mark.parametrize("args", [
    (X, 0, G, BETA, Y, H_, 4, 8, 1e-5, None, None, None),        # null r
    (X, R_, G, BETA, Y, Y, 4, 8, 1e-5, None, None, None),        # h == y
    (X, R_, G, BETA, Y, Y + 16, 4, 8, 1e-5, None, None, None),   # h overlaps y
    (X, R_, G, BETA, Y, R_ + 4, 4, 8, 1e-5, None, None, None),   # h partially overlaps r
    (X, X + 8, G, BETA, Y, H_, 4, 8, 1e-5, None, None, None),    # r partially overlaps x
    (X, R_ + 2, G, BETA, Y, H_, 4, 8, 1e-5, None, None, None),   # r not 4-byte aligned
    (X, R_, Y + 64, BETA, Y, H_, 4, 8, 1e-5, None, None, None),  # gamma inside y
    (X, R_, G, BETA, Y, BETA, 4, 8, 1e-5, None, None, None),     # h over beta
])
def test_add_layernorm_rejects_bad_arguments(L, args):
    assert L.mi_add_layernorm_fwd(*args) == mn.MI_NORM_ERR_INVALID


@pytest.mark.parametrize("y,h", [(X, None), (R_, None), (X, R_), (R_, X), (Y, X), (Y, R_), (X, H_)])
def test_add_allowed_aliasing_is_accepted(L, y, h):
    # rows = 0 validates fully and launches nothing, so this runs without a device
    assert L.mi_add_layernorm_fwd(X, R_, G, BETA, y, h, 0, 8, 1e-5, None, None, None) == mn.MI_NORM_OK
    p = mn.problem(mn.OP_ADD_LAYERNORM, 4096, 768, X, y, G, BETA, r=R_, h=h)
    assert mn.mi_norm_select(p) >= 0


def test_add_rmsnorm_validation(L):
    assert L.mi_add_rmsnorm_fwd(X, R_, G, Y, H_, 0, 8, 1e-5, None, None) == mn.MI_NORM_OK
    assert L.mi_add_rmsnorm_fwd(X, 0, G, Y, H_, 4, 8, 1e-5, None, None) == mn.MI_NORM_ERR_INVALID
    assert L.mi_add_rmsnorm_fwd(X, R_, G, Y, Y, 4, 8, 1e-5, None, None) == mn.MI_NORM_ERR_INVALID
    assert L.mi_add_rmsnorm_fwd(X, R_, Y + 4, Y, H_, 4, 8, 1e-5, None, None) == mn.MI_NORM_ERR_INVALID


# --- variant table and dispatch (host logic) ---------------------------------

OPS = (mn.OP_LAYERNORM, mn.OP_RMSNORM, mn.OP_ADD_LAYERNORM, mn.OP_ADD_RMSNORM)
PREFIX = {mn.OP_LAYERNORM: "ln_", mn.OP_RMSNORM: "rms_", mn.OP_ADD_LAYERNORM: "addln_",
          mn.OP_ADD_RMSNORM: "addrms_"}


def _infos():
    return [(i, mn.mi_norm_variant_name(i), mn.mi_norm_variant_get_info(i))
            for i in range(mn.mi_norm_variant_count())]


def _prob(op, rows, d, x=X, y=Y, g=G, b=BETA, r=R_, h=H_):
    add = op >= mn.OP_ADD_LAYERNORM
    ln = op in (mn.OP_LAYERNORM, mn.OP_ADD_LAYERNORM)
    return mn.problem(op, rows, d, x, y, g, b if ln else None, r=r if add else None,
                      h=h if add else None)


def test_select_rejects_invalid_problems(L):
    assert mn.mi_norm_select(_prob(0, -1, 768)) == -1
    assert mn.mi_norm_select(_prob(7, 16, 768)) == -1
    assert mn.mi_norm_select(_prob(mn.OP_ADD_LAYERNORM, 16, 768, r=None)) == -1
    assert L.mi_norm_select(None) == -1


def test_variant_table_is_consistent(L):
    infos = _infos()
    names = [n for _, n, _ in infos]
    assert len(set(names)) == len(names)
    assert mn.mi_norm_variant_name(len(infos)) is None
    assert mn.mi_norm_variant_name(-1) is None
    for i, n, v in infos:
        assert n.startswith(PREFIX[v["op"]]), n
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
    assert {v["op"] for _, _, v in infos} == set(OPS)
    # every operation has the same family of shapes
    shapes = {op: sorted(n[len(PREFIX[op]):] for _, n, v in infos if v["op"] == op) for op in OPS}
    assert shapes[0] == shapes[1] == shapes[2] == shapes[3]


WIDTHS = sorted({1, 2, 3, 4, 5, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 255, 256,
                 257, 511, 512, 513, 767, 768, 769, 1000, 1023, 1024, 1025, 2047, 2048, 2049, 3000,
                 3072, 4095, 4096, 4097, 6144, 8191, 8192, 8193, 12288, 16383, 16384, 16385, 32767,
                 32768, 32769, 65536, 100003, 2**20})


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("layout", ["aligned", "same_phase", "different_phase"])
def test_dispatch_picks_an_eligible_covering_variant(L, op, layout):
    if layout == "aligned":
        ptrs = dict(x=X, y=Y, r=R_, h=H_)
    elif layout == "same_phase":
        ptrs = dict(x=X + 4, y=Y + 4, r=R_ + 4, h=H_ + 4)
    else:
        ptrs = dict(x=X + 4, y=Y + 8, r=R_ + 4, h=H_ + 4)
    for rows in (64, 4096):
        for d in WIDTHS:
            p = _prob(op, rows, d, **ptrs)
            vid = mn.mi_norm_select(p)
            assert vid >= 0, (op, d, layout)
            v = mn.mi_norm_variant_get_info(vid)
            assert v["op"] == op
            assert mn.mi_norm_eligible(vid, p), (d, layout, mn.mi_norm_variant_name(vid))
            assert v["looped"] or v["max_d"] >= d
            if layout == "aligned" and d % 4 == 0:
                assert v["vec"] == 4 and not v["peel"], (d, mn.mi_norm_variant_name(vid))
            if layout == "different_phase":
                assert v["vec"] == 1, (d, mn.mi_norm_variant_name(vid))
            if layout == "aligned" and d % 4 and 256 <= d <= 32768:
                assert v["peel"], (d, mn.mi_norm_variant_name(vid))


def test_residual_pointers_decide_the_layout(L):
    # a residual or sum of another 16-byte phase takes the 32-bit path
    v = mn.mi_norm_variant_get_info(mn.mi_norm_select(_prob(mn.OP_ADD_LAYERNORM, 4096, 768, r=R_ + 4)))
    assert v["vec"] == 1
    v = mn.mi_norm_variant_get_info(mn.mi_norm_select(_prob(mn.OP_ADD_LAYERNORM, 4096, 768, h=H_ + 8)))
    assert v["vec"] == 1
    # without h, only x, r and y matter
    v = mn.mi_norm_variant_get_info(mn.mi_norm_select(_prob(mn.OP_ADD_RMSNORM, 4096, 768, h=None)))
    assert v["vec"] == 4 and not v["peel"]


def test_dispatch_examples(L):
    sel = lambda op, d, rows=4096, **k: mn.mi_norm_variant_name(mn.mi_norm_select(_prob(op, rows, d, **k)))
    assert sel(0, 768) == "ln_4_p0_l64_w1_q3_b16"            # 256 workgroups of 16 rows
    assert sel(0, 768, rows=1000) == "ln_4_p0_l64_w2_q2_b4"  # few rows: two waves per row
    assert sel(0, 2048, rows=1024) == "ln_4_p0_l64_w4_q2_b4"
    assert sel(0, 4096, rows=4096) == "ln_4_p0_l64_w4_q4_b16"
    assert sel(0, 8192, rows=32768) == "ln_4_p0_l64_w8_q4_b16"
    assert sel(0, 128, rows=512) == "ln_4_p0_l32_w1_q1_b4"
    assert sel(1, 8193, rows=256) == "rms_4_p1_l64_w16_q3_b16"
    assert sel(0, 1, rows=64) == "ln_1_p0_l16_w1_q1_b4"
    assert sel(2, 768) == "addln_4_p0_l64_w1_q3_b16"
    assert sel(3, 8192, rows=32768) == "addrms_4_p0_l64_w8_q4_b16"
    assert "_loop_" in sel(0, 2**20)
    # gamma misaligned only: no 128-bit parameter reads, so not the aligned path
    assert mn.mi_norm_variant_get_info(mn.mi_norm_select(_prob(0, 4096, 768, g=G + 4)))["needs_aligned"] == 0


def test_workgroup_size_follows_row_count(L):
    for d in (768, 2048, 4096, 8192, 16384):
        for rows in (1, 100, 1000, 5000, 100000):
            v = mn.mi_norm_variant_get_info(mn.mi_norm_select(_prob(0, rows, d)))
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
        v = mn.mi_norm_variant_get_info(mn.mi_norm_select(_prob(0, rows, d)))
        assert (v["waves_per_row"], v["slots"]) == (wpr, q), (d, rows, v)


def test_eligibility_rules(L):
    for i, n, v in _infos():
        op = v["op"]
        other = {0: 1, 1: 0, 2: 3, 3: 2}[op]
        assert not mn.mi_norm_eligible(i, _prob(other, 16, 64))
        if v["needs_aligned"]:
            assert not mn.mi_norm_eligible(i, _prob(op, 16, 64, x=X + 4))
            assert not mn.mi_norm_eligible(i, _prob(op, 16, 6))
        if not v["looped"]:
            assert not mn.mi_norm_eligible(i, _prob(op, 16, v["max_d"] + 4))
    assert not mn.mi_norm_eligible(-1, _prob(0, 16, 8))
    assert L.mi_layernorm_fwd_variant(10**6, X, G, BETA, Y, 4, 8, 1e-5, None, None, None) == mn.MI_NORM_ERR_INVALID
