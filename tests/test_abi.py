"""The C ABI on the CPU: the library loads, exports what the header declares,
rejects bad arguments before touching a device, and its dispatcher picks an
eligible variant for every width, storage type, stride and layout.  No kernel
is launched here: the addresses below are fake, so the module skips itself
where a GPU is visible."""
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
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-logic tests pass fake device addresses; run them where no GPU is visible")
    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return mn.lib()


def test_exports_every_declared_symbol(L):
    declared = B.header_functions()
    assert {"mi_layernorm_fwd", "mi_rmsnorm_fwd", "mi_norm_status_string"} <= set(declared)
    for name in declared:
        assert hasattr(L, name), f"{name} declared in mi_norm.h or mi_norm_tuning.h but not exported"
    nm = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True,
                        check=True).stdout
    exported = {l.split()[-1] for l in nm.splitlines() if " T " in l and l.split()[-1].startswith("mi_")}
    assert exported == set(declared), exported ^ set(declared)


def test_public_header_holds_the_interface_only():
    """mi_norm.h declares the operations and their checks; the variant table,
    forced variants and calibration kernels live in mi_norm_tuning.h."""
    public = set(B.header_functions(B.HEADER))
    tuning = set(B.header_functions(B.TUNING_HEADER))
    assert public == {
        "mi_norm_status_string", "mi_norm_version", "mi_layernorm_fwd", "mi_rmsnorm_fwd",
        "mi_add_layernorm_fwd", "mi_add_rmsnorm_fwd", "mi_norm_fwd", "mi_norm_check",
        "mi_norm_bwd_workspace_size", "mi_norm_bwd", "mi_norm_bwd_check", "mi_layernorm_bwd",
        "mi_rmsnorm_bwd", "mi_norm_bwd_noalloc", "mi_norm_bwd_noalloc_limit"}, public
    assert not public & tuning
    assert {"mi_norm_select", "mi_norm_fwd_variant", "mi_norm_bwd_variant", "mi_copy_f32",
            "mi_calib_launch"} <= tuning


@pytest.mark.parametrize("header", ["mi_norm.h", "mi_norm_tuning.h"])
def test_header_compiles_as_plain_c(header):
    r = subprocess.run(["gcc", "-std=c99", "-fsyntax-only", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-x", "c",
                        os.path.join(ROOT, "include", header)],
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


def test_row_geometry_of_torch_layouts():
    """The row count and stride the torch conveniences hand the C ABI, from a
    tensor's shape and strides; rows that repeat one another (stride 0, as
    in the upstream gradient of a sum over rows) are refused rather than
    passed as a stride of 0, which the ABI reads as d, and the binding
    copies such an input before it reaches the ABI."""
    import torch
    assert B._row_geometry((4096, 768), (768, 1), "x") == (4096, 768)
    assert B._row_geometry((64, 768), (1024, 1), "x") == (64, 1024)       # column slice
    assert B._row_geometry((3, 97, 768), (97 * 1024, 1024, 1), "x") == (291, 1024)
    assert B._row_geometry((1, 5, 768), (0, 768, 1), "x") == (5, 768)      # size-1 dims carry no stride
    assert B._row_geometry((768,), (1,), "x") == (1, 768)
    for shape, strides in (((64, 768), (0, 1)), ((2, 3, 768), (0, 0, 1)), ((2, 3, 768), (768, 0, 1))):
        with pytest.raises(ValueError, match="repeat"):
            B._row_geometry(shape, strides, "dy")
    with pytest.raises(ValueError):
        B._row_geometry((64, 768), (768, 2), "x")                          # last dimension strided
    with pytest.raises(ValueError):
        B._row_geometry((2, 3, 768), (4 * 768, 768 + 1, 1), "x")           # no single row stride
    # the loss sum(0)-then-square hands backward a dy of strides (0, 1)
    dy = torch.ones(768).expand(64, 768)
    assert dy.stride() == (0, 1)
    fixed = B._input_rows(dy)
    assert fixed.is_contiguous() and torch.equal(fixed, dy)
    plain = torch.zeros(64, 1024)[:, :768]
    assert B._input_rows(plain) is plain and B._input_rows(None) is None


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
    (X, R_, G, BETA, Y, X + 8, 4, 8, 1e-5, None, None, None),    # h partially overlaps x
    (X, R_, G, BETA, R_ + 4, H_, 4, 8, 1e-5, None, None, None),  # y partially overlaps r
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


def _prob(op, rows, d, x=X, y=Y, g=G, b=BETA, r=R_, h=H_, **kw):
    add = op >= mn.OP_ADD_LAYERNORM
    ln = op in (mn.OP_LAYERNORM, mn.OP_ADD_LAYERNORM)
    return mn.problem(op, rows, d, x, y, g, b if ln else None, r=r if add else None,
                      h=h if add else None, **kw)


def test_select_rejects_invalid_problems(L):
    assert mn.mi_norm_select(_prob(0, -1, 768)) == -1
    assert mn.mi_norm_select(_prob(7, 16, 768)) == -1
    assert mn.mi_norm_select(_prob(mn.OP_ADD_LAYERNORM, 16, 768, r=None)) == -1
    assert L.mi_norm_select(None) == -1


DTYPES = (mn.MI_NORM_F32, mn.MI_NORM_F16, mn.MI_NORM_BF16)
DTSFX = {mn.MI_NORM_F32: "", mn.MI_NORM_F16: "f16_", mn.MI_NORM_BF16: "bf16_"}
ESIZE = {mn.MI_NORM_F32: 4, mn.MI_NORM_F16: 2, mn.MI_NORM_BF16: 2}


BWD_PREFIX = {mn.OP_LAYERNORM_BWD: "lnbwd_", mn.OP_RMSNORM_BWD: "rmsbwd_"}


def test_variant_table_is_consistent(L):
    everything = _infos()
    names = [n for _, n, _ in everything]
    assert len(set(names)) == len(names)
    assert mn.mi_norm_variant_name(len(everything)) is None
    assert mn.mi_norm_variant_name(-1) is None
    infos = [t for t in everything if t[2]["op"] in OPS]
    bwd = [t for t in everything if t[2]["op"] in BWD_PREFIX]
    assert len(infos) + len(bwd) == len(everything)
    # forward ids first, then backward
    assert max(i for i, _, _ in infos) < min(i for i, _, _ in bwd)
    for i, n, v in bwd:
        assert n.startswith(BWD_PREFIX[v["op"]] + DTSFX[v["dtype"]]), n
        assert v["lanes_per_row"] == 64 and not v["peel"] and v["rows_per_lane"] == 1
        if v["looped"]:
            assert v["max_d"] == 2**63 - 1 and v["vec"] in (1, 16 // ESIZE[v["dtype"]])
            assert v["needs_aligned"] == (1 if v["vec"] > 1 else 0)
            continue
        assert v["rows_per_block"] * v["waves_per_row"] == v["waves_per_block"]
        assert v["waves_per_block"] == 8 and n.endswith("_b8"), n
        assert v["max_d"] == v["vec"] * 64 * v["waves_per_row"] * v["slots"]
        assert v["needs_aligned"] == (1 if v["vec"] > 1 else 0)
        assert v["vec"] in (1, 16 // ESIZE[v["dtype"]])
        # LayerNorm lanes hold at most 24 vector values, RMSNorm 32
        if v["vec"] > 1:
            assert v["vec"] * v["slots"] <= (24 if v["op"] == mn.OP_LAYERNORM_BWD else 32), n
    assert {(v["op"], v["dtype"]) for _, _, v in bwd} == {(o, t) for o in BWD_PREFIX for t in DTYPES}
    for i, n, v in infos:
        assert n.startswith(PREFIX[v["op"]] + DTSFX[v["dtype"]]), n
        if v["dtype"] == mn.MI_NORM_F32:
            assert "f16_" not in n, n
        if v["looped"]:
            assert v["max_d"] == 2**63 - 1 and v["rows_per_block"] == 1
            continue
        # a peeled row holds its head and tail apart from the body
        assert v["max_d"] == v["vec"] * v["lanes_per_row"] * v["waves_per_row"] * v["slots"] + (
            v["vec"] - 1 if v["peel"] else 0)
        assert v["rows_per_lane"] in (1, 2), n
        if v["rows_per_lane"] == 2:
            # multi-row: aligned vector path, full-wave rows, two rows per wave group
            assert "_r2_" in n and v["vec"] > 1 and not v["peel"] and v["lanes_per_row"] == 64, n
            assert v["rows_per_block"] == 2 * v["waves_per_block"] // v["waves_per_row"], n
            assert v["waves_per_row"] <= 8 and v["slots"] <= (8 if v["vec"] == 4 else 4), n
        elif v["waves_per_row"] == 1:
            assert v["rows_per_block"] == v["waves_per_block"] * 64 // v["lanes_per_row"]
        else:
            assert v["lanes_per_row"] == 64
            assert v["rows_per_block"] * v["waves_per_row"] == v["waves_per_block"]
        assert v["waves_per_block"] * 64 <= 1024
        assert v["needs_aligned"] == (1 if v["vec"] > 1 and not v["peel"] else 0)
        # vector accesses are 16 bytes: 4 float32 or 8 16-bit elements
        assert v["vec"] in (1, 16 // ESIZE[v["dtype"]])
    assert {v["op"] for _, _, v in infos} == set(OPS)
    assert {v["dtype"] for _, _, v in infos} == set(DTYPES)
    # within a storage type every operation has the same family of shapes,
    # and the two 16-bit types have the same family; float32 LayerNorm alone
    # adds one wave per row with sixteen slots (4- and 8-wave workgroups)
    shapes = {(op, dt): sorted(n[len(PREFIX[op] + DTSFX[dt]):] for _, n, v in infos
                               if v["op"] == op and v["dtype"] == dt) for op in OPS for dt in DTYPES}
    wide16 = ["4_p0_l64_w1_q16_b4", "4_p0_l64_w1_q16_b8", "4_p0_l64_w1_q16_b16"]
    assert all(w in shapes[(0, mn.MI_NORM_F32)] for w in wide16)
    shapes[(0, mn.MI_NORM_F32)] = [n for n in shapes[(0, mn.MI_NORM_F32)] if n not in wide16]
    for dt in DTYPES:
        assert shapes[(0, dt)] and all(shapes[(op, dt)] == shapes[(0, dt)] for op in OPS)
    assert shapes[(0, mn.MI_NORM_F16)] == shapes[(0, mn.MI_NORM_BF16)]
    # float32 ids come first, so they do not move when other types are added
    assert [v["dtype"] for _, _, v in infos] == sorted(v["dtype"] for _, _, v in infos)


WIDTHS = sorted({1, 2, 3, 4, 5, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 255, 256,
                 257, 511, 512, 513, 767, 768, 769, 1000, 1023, 1024, 1025, 2047, 2048, 2049, 3000,
                 3072, 4095, 4096, 4097, 6144, 8191, 8192, 8193, 12288, 16383, 16384, 16385, 32767,
                 32768, 32769, 65536, 100003, 2**20})


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("layout", ["aligned", "same_phase", "different_phase"])
def test_dispatch_picks_an_eligible_covering_variant(L, op, layout, dt):
    e = ESIZE[dt]
    if layout == "aligned":
        ptrs = dict(x=X, y=Y, r=R_, h=H_)
    elif layout == "same_phase":
        ptrs = dict(x=X + e, y=Y + e, r=R_ + e, h=H_ + e)
    else:
        ptrs = dict(x=X + e, y=Y + 2 * e, r=R_ + e, h=H_ + e)
    for rows in (64, 4096):
        for d in WIDTHS:
            p = _prob(op, rows, d, dtype=dt, **ptrs)
            vid = mn.mi_norm_select(p)
            assert vid >= 0, (op, d, layout)
            v = mn.mi_norm_variant_get_info(vid)
            assert v["op"] == op and v["dtype"] == dt
            assert mn.mi_norm_eligible(vid, p), (d, layout, mn.mi_norm_variant_name(vid))
            assert v["looped"] or v["max_d"] >= d
            W = 16 // e
            if layout == "aligned" and d % W == 0:
                assert v["vec"] == W and not v["peel"], (d, mn.mi_norm_variant_name(vid))
            if layout == "different_phase":
                assert v["vec"] == 1, (d, mn.mi_norm_variant_name(vid))
            if layout == "aligned" and d % W and 256 <= d <= (32768 if W == 4 else 49152):
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
    assert sel(0, 2048, rows=4096) == "ln_4_p0_l64_w2_q4_b16"  # 32 MiB: one row per wave
    # float32 LayerNorm rows of 3-4 K elements, 3072-4096 rows: one wave per
    # row with sixteen slots, in workgroups that fill whole rounds
    assert sel(0, 4096, rows=4096) == "ln_4_p0_l64_w1_q16_b8"
    assert sel(0, 3584, rows=3500) == "ln_4_p0_l64_w1_q16_b8"
    assert sel(0, 4096, rows=3072) == "ln_4_p0_l64_w1_q16_b4"
    assert sel(0, 4096, rows=3071) == "ln_4_p0_l64_w2_q8_b4"
    assert sel(0, 3072, rows=4096) == "ln_4_p0_l64_w2_q6_b16"
    assert sel(1, 4096, rows=4096) == "rms_4_r2_w4_q4_b4"
    assert sel(1, 4096, rows=8192) == "rms_4_r2_w4_q4_b4"         # many rows: two rows per wave group
    # float32 one-row path with more than 4096 waves at half the waves per
    # row: half the waves, twice the slots
    assert sel(1, 4096, rows=3072) == "rms_4_p0_l64_w2_q8_b4"
    assert sel(0, 2048, rows=6144) == "ln_4_p0_l64_w1_q8_b4"     # 16-wave grid uneven: 4 waves
    assert sel(0, 4096, rows=2048) == "ln_4_p0_l64_w4_q4_b16"    # 4096 waves: no change
    assert sel(2, 4096, rows=3000) == "addln_4_r2_w2_q8_b4"       # fused rows: their own rule
    # workgroups spread evenly over the CUs: 384 16-wave workgroups would load
    # half the CUs twice, so 4-wave ones
    assert sel(0, 768, rows=6144) == "ln_4_p0_l64_w1_q3_b4"
    assert sel(1, 768, rows=5000) == "rms_4_p0_l64_w1_q3_b4"
    assert sel(0, 768, rows=4096) == "ln_4_p0_l64_w1_q3_b16"
    # from 8192 rows or 64 MiB of rows, two rows per wave group
    assert sel(0, 4096, rows=4097) == "ln_4_r2_w4_q4_b4"
    assert sel(0, 8192, rows=32768) == "ln_4_r2_w8_q4_b8"
    assert sel(0, 768, rows=8192) == "ln_4_r2_w1_q3_b4"
    assert sel(0, 768, rows=8191) == "ln_4_p0_l64_w1_q3_b16"
    # one wave per row on rows 3.5 KiB or more apart: two rows per wave group
    assert sel(0, 1024, rows=4096) == "ln_4_r2_w1_q4_b4"
    assert sel(0, 896, rows=4096) == "ln_4_r2_w1_q4_b4"
    assert sel(0, 768, rows=4096, ldx=1024, ldy=1024) == "ln_4_r2_w1_q3_b4"
    assert sel(0, 768, rows=4096, ldx=880) == "ln_4_p0_l64_w1_q3_b16"
    # 16-bit rows of one or two waves: one row per wave group, parameters in LDS
    assert sel(0, 2048, rows=4096, dtype=mn.MI_NORM_BF16) == "ln_bf16_8_p0_l64_w1_q4_b4"
    assert sel(0, 2048, rows=32768, dtype=mn.MI_NORM_F16) == "ln_f16_8_p0_l64_w1_q4_b4"
    assert sel(2, 768, rows=8192, dtype=mn.MI_NORM_BF16) == "addln_bf16_8_p0_l64_w1_q2_b4"
    # plain 16-bit rows of one or two slots up to 8192 rows: the workgroup rule
    assert sel(0, 768, rows=8192, dtype=mn.MI_NORM_BF16) == "ln_bf16_8_p0_l64_w1_q2_b16"
    assert sel(0, 768, rows=16384, dtype=mn.MI_NORM_BF16) == "ln_bf16_8_p0_l64_w1_q2_b4"
    assert sel(0, 768, rows=2048, dtype=mn.MI_NORM_BF16) == "ln_bf16_8_p0_l64_w1_q2_b4"
    # with 2560-8192 rows, rows of two waves run as one wave with twice the
    # slots in 16-wave workgroups
    assert sel(1, 4096, rows=8192, dtype=mn.MI_NORM_BF16) == "rms_bf16_8_p0_l64_w1_q8_b16"
    assert sel(0, 4096, rows=2560, dtype=mn.MI_NORM_BF16) == "ln_bf16_8_p0_l64_w1_q8_b16"
    assert sel(2, 3072, rows=4096, dtype=mn.MI_NORM_F16) == "addln_f16_8_p0_l64_w1_q6_b16"
    # fused float32 rows of four waves, 2048-4095 rows: multi-row, two waves,
    # twice the slots
    assert sel(2, 3000, rows=3000) == "addln_4_r2_w2_q6_b4"
    assert sel(3, 4096, rows=2048) == "addrms_4_r2_w2_q8_b4"
    assert sel(2, 3072, rows=4096) == "addln_4_r2_w4_q3_b4"
    # ... in 4-wave workgroups where more than 256 16-wave ones spread unevenly
    assert sel(0, 3000, rows=5000, dtype=mn.MI_NORM_BF16) == "ln_bf16_8_p0_l64_w1_q6_b4"
    assert sel(0, 3072, rows=8000, dtype=mn.MI_NORM_BF16) == "ln_bf16_8_p0_l64_w1_q6_b16"   # 500: even
    # fused 16-bit rows of two waves and four slots, 4097-8192 rows: four waves
    assert sel(2, 4096, rows=8000, dtype=mn.MI_NORM_BF16) == "addln_bf16_8_p0_l64_w4_q2_b16"
    assert sel(3, 4096, rows=4096, dtype=mn.MI_NORM_BF16) == "addrms_bf16_8_p0_l64_w1_q8_b16"
    # fused 16-bit rows of four waves keep four waves from 2560 rows
    assert sel(3, 6000, rows=3000, dtype=mn.MI_NORM_BF16) == "addrms_bf16_8_p0_l64_w4_q3_b16"
    assert sel(2, 6144, rows=2048, dtype=mn.MI_NORM_BF16) == "addln_bf16_8_p0_l64_w2_q6_b16"
    # float32 RMSNorm rows of two waves, 2048-4096 rows: the base shape (the
    # multi-row kernel won by 5-6% there, under the box-to-box spread)
    assert sel(1, 2048, rows=2560) == "rms_4_p0_l64_w2_q4_b4"
    assert sel(1, 1536, rows=4096) == "rms_4_p0_l64_w2_q3_b16"
    assert sel(0, 2048, rows=4096) == "ln_4_p0_l64_w2_q4_b16"
    # fused float32 rows of two waves up to 4096 rows: one wave of eight slots
    assert sel(2, 1536, rows=2048) == "addln_4_p0_l64_w1_q8_b4"
    assert sel(3, 2048, rows=4096) == "addrms_4_p0_l64_w1_q8_b4"
    assert sel(2, 2048, rows=4097) == "addln_4_r2_w2_q4_b4"
    assert sel(2, 1028, rows=4096) == "addln_4_p0_l64_w1_q8_b4"       # 257 quads
    assert sel(2, 1024, rows=4096) == "addln_4_r2_w1_q4_b4"           # one wave by width
    # under 2560 rows, rows of two waves and three or four slots: multi-row
    assert sel(1, 4096, rows=2048, dtype=mn.MI_NORM_BF16) == "rms_bf16_8_r2_w2_q4_b4"
    assert sel(3, 4096, rows=2559, dtype=mn.MI_NORM_BF16) == "addrms_bf16_8_r2_w2_q4_b4"
    assert sel(0, 3072, rows=2048, dtype=mn.MI_NORM_F16) == "ln_f16_8_r2_w2_q3_b4"
    assert sel(0, 2048, rows=2048, dtype=mn.MI_NORM_BF16) == "ln_bf16_8_p0_l64_w2_q2_b4"   # two slots
    assert sel(0, 4096, rows=1024, dtype=mn.MI_NORM_BF16) == "ln_bf16_8_p0_l64_w4_q2_b4"   # four waves
    assert sel(0, 4096, rows=8193, dtype=mn.MI_NORM_BF16) == "ln_bf16_8_p0_l64_w2_q4_b4"
    # from four waves per row, the 16-bit rows follow the float32 rules
    assert sel(0, 8192, rows=32768, dtype=mn.MI_NORM_BF16) == "ln_bf16_8_r2_w4_q4_b4"
    assert sel(0, 8192, rows=4096, dtype=mn.MI_NORM_BF16) == "ln_bf16_8_r2_w4_q4_b4"   # 64 MiB
    # 16-bit rows of four waves on the one-row path from 2048 rows: two waves,
    # twice the slots, 16-wave workgroups
    assert sel(0, 8192, rows=4095, dtype=mn.MI_NORM_BF16) == "ln_bf16_8_p0_l64_w2_q8_b16"
    assert sel(1, 6144, rows=4096, dtype=mn.MI_NORM_F16) == "rms_f16_8_p0_l64_w2_q6_b16"
    assert sel(3, 8192, rows=2048, dtype=mn.MI_NORM_BF16) == "addrms_bf16_8_p0_l64_w2_q8_b16"
    assert sel(0, 8192, rows=2047, dtype=mn.MI_NORM_BF16) == "ln_bf16_8_p0_l64_w4_q4_b16"
    # no multi-row variant for 16 waves per row, or for more than 4 slots of 16-bit rows
    assert sel(0, 16384, rows=8192) == "ln_4_p0_l64_w16_q4_b16"
    assert sel(0, 6144 * 8, rows=8192, dtype=mn.MI_NORM_BF16) == "ln_bf16_8_p0_l64_w16_q6_b16"
    assert sel(0, 128, rows=512) == "ln_4_p0_l32_w1_q1_b4"
    # a peeled row's body holds at most d / 4 accesses: 8193 fits 16 waves of two
    assert sel(1, 8193, rows=256) == "rms_4_p1_l64_w16_q2_b16"
    # peeled rows of fewer than eight waves keep the fewest waves that hold
    # them in four slots, in the largest workgroups that still give every CU one
    assert sel(0, 2049, rows=1024) == "ln_4_p1_l64_w2_q4_b4"
    assert sel(1, 4097, rows=1024) == "rms_4_p1_l64_w4_q4_b16"
    assert sel(0, 1025, rows=2048) == "ln_4_p1_l64_w1_q4_b4"
    assert sel(0, 8193, rows=512) == "ln_4_p1_l64_w8_q4_b16"
    assert sel(0, 4100, rows=1024, dtype=mn.MI_NORM_BF16) == "ln_bf16_8_p1_l64_w2_q4_b4"
    assert sel(0, 1, rows=64) == "ln_1_p0_l16_w1_q1_b4"
    assert sel(2, 768) == "addln_4_r2_w1_q3_b4"             # fused: two rows per wave group
    assert sel(2, 768, rows=4095) == "addln_4_p0_l64_w2_q2_b16"
    # fused rows of four or eight waves with many rows: one row per wave group,
    # twice the waves and half the slots
    assert sel(3, 8192, rows=32768) == "addrms_4_p0_l64_w16_q2_b16"
    assert sel(2, 4096, rows=16384) == "addln_4_p0_l64_w8_q2_b16"
    assert sel(2, 8192, rows=32768, dtype=mn.MI_NORM_BF16) == "addln_bf16_8_p0_l64_w8_q2_b16"
    assert sel(2, 6144, rows=16384) == "addln_4_p0_l64_w16_q2_b16"
    assert sel(2, 4096, rows=8191) == "addln_4_r2_w4_q4_b4"      # fewer rows: two rows per wave group
    assert "_loop_" in sel(0, 2**20)
    # gamma misaligned only: no 128-bit parameter reads, so not the aligned path
    assert mn.mi_norm_variant_get_info(mn.mi_norm_select(_prob(0, 4096, 768, g=G + 4)))["needs_aligned"] == 0


def test_workgroup_size_follows_row_count(L):
    for d in (768, 2048, 4096, 8192, 16384):
        for rows in (1, 100, 1000, 5000, 100000):
            v = mn.mi_norm_variant_get_info(mn.mi_norm_select(_prob(0, rows, d)))
            if v["rows_per_lane"] == 2:
                # multi-row variants have a fixed workgroup: 4 waves, 8 at 8 waves per row
                assert rows >= 8192 or rows * d * 4 >= 64 << 20 or (v["waves_per_row"] == 1 and 4 * d >= 3584), \
                    (d, rows)
                assert v["waves_per_block"] == max(4, v["waves_per_row"]), (d, rows)
                continue
            need = 512 if v["waves_per_row"] > 1 else 256
            per16 = 16 // v["waves_per_row"]
            even = lambda blocks: -(-blocks // 256) * 256 * 100 <= blocks * 115
            if v["waves_per_block"] < 16:
                # a 16-wave workgroup would have left too few workgroups, or
                # spread them unevenly over the 256 CUs
                b16 = -(-rows // per16)
                assert b16 < need or not even(b16), (d, rows)
            else:
                blocks = -(-rows // v["rows_per_block"])
                assert (blocks >= need and even(blocks)) or v["waves_per_row"] == 16, (d, rows)


def test_rows_spread_over_more_waves_when_few(L):
    # about four accesses per lane with many rows (float32 one-row rows of
    # 2-4 K elements: up to eight); more waves per row with few
    for d, rows, wpr, q in ((768, 4096, 1, 3), (2048, 4096, 2, 4), (2048, 1024, 4, 2),
                            (4096, 8192, 4, 4), (4096, 2048, 4, 4), (8192, 32768, 8, 4), (16384, 8192, 16, 4),
                            (768, 100, 2, 2), (32768, 64, 16, 8)):
        v = mn.mi_norm_variant_get_info(mn.mi_norm_select(_prob(0, rows, d)))
        assert (v["waves_per_row"], v["slots"]) == (wpr, q), (d, rows, v)


def test_eligibility_rules(L):
    for i, n, v in _infos():
        op, dt = v["op"], v["dtype"]
        if op not in OPS:
            continue                     # backward variants: test_bwd_dispatch_covers_every_width
        other = {0: 1, 1: 0, 2: 3, 3: 2}[op]
        assert not mn.mi_norm_eligible(i, _prob(other, 16, 64, dtype=dt))
        assert not mn.mi_norm_eligible(i, _prob(op, 16, 64, dtype=(dt + 1) % 3))
        if v["needs_aligned"]:
            assert not mn.mi_norm_eligible(i, _prob(op, 16, 64, x=X + ESIZE[dt], dtype=dt))
            assert not mn.mi_norm_eligible(i, _prob(op, 16, 6, dtype=dt))
            assert not mn.mi_norm_eligible(i, _prob(op, 16, 64, ldx=66, dtype=dt))
        if not v["looped"]:
            assert not mn.mi_norm_eligible(i, _prob(op, 16, v["max_d"] + 4, dtype=dt))
    assert not mn.mi_norm_eligible(-1, _prob(0, 16, 8))
    assert L.mi_layernorm_fwd_variant(10**6, X, G, BETA, Y, 4, 8, 1e-5, None, None, None) == mn.MI_NORM_ERR_INVALID


# --- storage types, row strides and the general call --------------------------

def _check(op=mn.OP_LAYERNORM, rows=4, d=8, **kw):
    return mn.mi_norm_check(_prob(op, rows, d, **kw))


def test_general_call_validation(L):
    OK, BAD = mn.MI_NORM_OK, mn.MI_NORM_ERR_INVALID
    assert _check() == OK
    assert L.mi_norm_check(None) == BAD and L.mi_norm_fwd(None, None) == BAD
    assert _check(dtype=3) == BAD and _check(dtype=-1) == BAD
    assert _check(dtype=mn.MI_NORM_BF16, x=X + 2) == OK          # 2-byte aligned is enough
    assert _check(dtype=mn.MI_NORM_BF16, x=X + 1) == BAD
    assert _check(dtype=mn.MI_NORM_F32, x=X + 2) == BAD
    assert _check(ldx=7) == BAD and _check(ldy=-8) == BAD          # stride below d, negative
    assert _check(ldx=8, ldy=0) == OK and _check(ldx=1000, ldy=12) == OK
    assert _check(rows=1, ldx=3) == OK                             # one row: no stride is used
    assert _check(rows=2**40, d=8, ldx=2**30) == BAD               # extent overflows
    assert _check(eps=float("nan")) == BAD
    assert _check(mean=0x7F0600000000 + 2) == BAD                  # misaligned statistics
    assert _check(op=mn.OP_RMSNORM, b=None, mean=X) == OK          # RMSNorm ignores mean
    assert _check(mean=X + 4) == BAD                               # mean inside x
    assert _check(mean=0x7F0600000000, rstd=0x7F0600000000 + 8) == BAD   # mean meets rstd
    assert _check(rstd=G) == BAD                                   # rstd over gamma


def test_strided_aliasing_is_exact_for_equal_strides(L):
    OK, BAD = mn.MI_NORM_OK, mn.MI_NORM_ERR_INVALID
    d, ld = 8, 16
    # y interleaved with x in one [rows, 2d] buffer: no shared element
    assert _check(d=d, x=X, y=X + 4 * d, ldx=ld, ldy=ld) == OK
    assert _check(d=d, x=X + 4 * d, y=X, ldx=ld, ldy=ld) == OK
    # one element off: the rows overlap
    assert _check(d=d, x=X, y=X + 4 * (d - 1), ldx=ld, ldy=ld) == BAD
    assert _check(d=d, x=X, y=X + 4 * (d + 1), ldx=ld, ldy=ld) == BAD   # y's row runs into x's next row
    # in place needs the same stride
    assert _check(d=d, x=X, y=X, ldx=ld, ldy=ld) == OK
    assert _check(d=d, x=X, y=X, ldx=ld, ldy=d) == BAD
    # different strides: any overlap of the extents is refused
    assert _check(d=d, x=X, y=X + 4 * d, ldx=ld, ldy=ld + 4) == BAD
    # inputs may share memory: x and r interleaved, or even the same tensor
    add = mn.OP_ADD_LAYERNORM
    assert _check(op=add, d=d, x=X, r=X + 4 * d, ldx=ld, ldr=ld, h=None) == OK
    assert _check(op=add, d=d, x=X, r=X + 4, h=None) == OK
    assert _check(op=add, d=d, x=X, r=X, h=None) == OK
    # y and h never share an element, and y may not be h
    assert _check(op=add, d=d, y=Y, h=Y + 4 * d, ldy=ld, ldh=ld) == OK
    assert _check(op=add, d=d, y=Y, h=Y, ldy=ld, ldh=ld) == BAD


def test_strides_and_types_decide_the_layout(L):
    info = lambda **kw: mn.mi_norm_variant_get_info(mn.mi_norm_select(_prob(0, 4096, 768, **kw)))
    name = lambda **kw: mn.mi_norm_variant_name(mn.mi_norm_select(_prob(0, 4096, 768, **kw)))
    # 16-byte accesses: eight 16-bit elements, 96 of them per row of 768
    assert name(dtype=mn.MI_NORM_BF16) == "ln_bf16_8_p0_l64_w1_q2_b16"
    assert name(dtype=mn.MI_NORM_F16) == "ln_f16_8_p0_l64_w1_q2_b16"
    assert info(dtype=mn.MI_NORM_BF16, x=X + 8, y=Y + 8)["peel"] == 1
    assert info(dtype=mn.MI_NORM_F32, x=X + 8, y=Y + 8)["peel"] == 1
    # a 16-bit row width that is a multiple of 4 but not of 8 is peeled
    v = mn.mi_norm_variant_get_info(mn.mi_norm_select(_prob(0, 4096, 772, dtype=mn.MI_NORM_BF16)))
    assert v["peel"] == 1 and v["vec"] == 8
    # peeled 16-bit rows stop at six slots (a body of 49152 elements, and a
    # head and tail of up to seven), then stream
    v = mn.mi_norm_variant_get_info(mn.mi_norm_select(_prob(2, 64, 49159, x=X + 2, y=Y + 2, r=R_ + 2,
                                                            h=H_ + 2, dtype=mn.MI_NORM_BF16)))
    assert v["peel"] == 1 and v["slots"] == 6
    v = mn.mi_norm_variant_get_info(mn.mi_norm_select(_prob(2, 64, 49160, x=X + 2, y=Y + 2, r=R_ + 2,
                                                            h=H_ + 2, dtype=mn.MI_NORM_BF16)))
    assert v["looped"] == 1 and v["vec"] == 1
    # strides that keep every row on a quad boundary keep the quad path
    assert info(ldx=1024, ldy=776)["needs_aligned"] == 1
    # a stride off the quad grid: rows change phase, together if all strides agree mod 4
    assert info(ldx=770, ldy=770)["peel"] == 1
    assert info(ldx=770, ldy=768)["vec"] == 1


def test_named_calls_equal_the_general_call(L):
    p = _prob(mn.OP_ADD_RMSNORM, 4096, 768, dtype=mn.MI_NORM_F32)
    assert mn.mi_norm_variant_name(mn.mi_norm_select(p)) == "addrms_4_r2_w1_q3_b4"
    assert L.mi_add_rmsnorm_fwd(X, R_, G, Y, Y, 4, 8, 1e-5, None, None) == mn.MI_NORM_ERR_INVALID
    assert mn.mi_norm_check(_prob(mn.OP_ADD_RMSNORM, 4, 8, h=Y)) == mn.MI_NORM_ERR_INVALID


# --- backward: validation, workspace and dispatch (host logic) ------------------

DY, DX, MEAN, RSTD, DG, DB, WS = (0x7F0700000000, 0x7F0800000000, 0x7F0900000000, 0x7F0A00000000,
                                  0x7F0B00000000, 0x7F0C00000000, 0x7F0D00000000)


def _bprob(op=mn.OP_LAYERNORM, rows=64, d=768, ws=WS, ws_bytes=None, **kw):
    ln = op == mn.OP_LAYERNORM
    args = dict(dy=DY, x=X, dx=DX, params0=G, mean=MEAN if ln else None, rstd=RSTD, dparams0=DG,
                dparams1=DB if ln else None)
    ptr_keys = set(args)
    args.update({k: v for k, v in kw.items() if k in ptr_keys})
    rest = {k: v for k, v in kw.items() if k not in ptr_keys}
    p = mn.bwd_problem(op, rows, d, args["dy"], args["x"], args["dx"], args["params0"], args["mean"], args["rstd"],
                       args["dparams0"], args["dparams1"], ws, 0, **rest)
    p.workspace_bytes = mn.mi_norm_bwd_workspace_size(p) if ws_bytes is None else ws_bytes
    return p


def test_bwd_workspace_size(L):
    p = _bprob(rows=4096, d=768)
    n = mn.mi_norm_bwd_workspace_size(p)
    # 256 partial rows of (dgamma, dbeta), then the per-row statistics; 256-byte sections
    assert n == 256 * 2 * 768 * 4 + 4096 * 8
    assert mn.mi_norm_bwd_workspace_size(_bprob(op=mn.OP_RMSNORM, rows=4096, d=768)) == 256 * 768 * 4 + 4096 * 8
    assert mn.mi_norm_bwd_workspace_size(_bprob(rows=3, d=5)) == 256 * 2 * 8 * 4 + 256
    # no parameter gradients: only the statistics section
    assert mn.mi_norm_bwd_workspace_size(_bprob(rows=100, d=64, dparams0=None, dparams1=None)) == 1024
    assert mn.mi_norm_bwd_workspace_size(_bprob(d=0)) == -1
    assert mn.mi_norm_bwd_workspace_size(_bprob(dtype=5)) == -1
    assert L.mi_norm_bwd_workspace_size(None) == -1


def test_widest_row(L):
    """The widest row accepted is 2^31 - 2^16 elements: the streamed-row
    kernels step an int32 element index by up to a few thousand past the
    row's end, which must stay representable.  Far-apart fake pointers keep
    8 GiB rows from overlapping; nothing is launched."""
    widest = 2**31 - 2**16
    x, y, g, b = 1 << 40, 1 << 41, 1 << 42, (1 << 42) + (1 << 36)
    for op in (mn.OP_LAYERNORM, mn.OP_RMSNORM, mn.OP_ADD_LAYERNORM):
        for d, want in ((widest, mn.MI_NORM_OK), (widest + 1, mn.MI_NORM_ERR_INVALID)):
            p = _prob(op, 1, d, x=x, y=y, g=g, b=b, r=1 << 43, h=None)
            assert mn.mi_norm_check(p) == want, (op, d)
    assert L.mi_rmsnorm_fwd(x, g, y, 1, widest + 1, 1e-5, None, None) == mn.MI_NORM_ERR_INVALID
    bw = dict(dy=1 << 40, x=1 << 41, dx=1 << 42, params0=(1 << 43), mean=(1 << 43) + (1 << 36),
              rstd=(1 << 43) + (1 << 37), dparams0=None, dparams1=None, ws=1 << 44, ws_bytes=1 << 20)
    assert mn.mi_norm_bwd_check(_bprob(rows=1, d=widest, **bw)) == mn.MI_NORM_OK
    assert mn.mi_norm_bwd_check(_bprob(rows=1, d=widest + 1, **bw)) == mn.MI_NORM_ERR_INVALID
    assert mn.mi_norm_bwd_workspace_size(_bprob(rows=1, d=widest + 1, **bw)) == -1


def test_bwd_validation(L):
    OK, BAD = mn.MI_NORM_OK, mn.MI_NORM_ERR_INVALID
    chk = lambda **kw: mn.mi_norm_bwd_check(_bprob(**kw))
    assert chk() == OK
    assert chk(op=mn.OP_RMSNORM) == OK
    assert chk(op=mn.OP_ADD_LAYERNORM) == BAD
    assert chk(mean=None) == BAD and chk(op=mn.OP_RMSNORM, mean=None) == OK
    assert chk(rstd=None) == BAD and chk(dy=None) == BAD and chk(dx=None) == BAD
    assert chk(ws=None) == BAD                       # parameter gradients need the workspace
    assert chk(ws=None, dparams0=None, dparams1=None) == OK   # dx alone at this width needs none
    assert chk(ws=WS + 64) == BAD                    # not 256-byte aligned
    assert chk(ws_bytes=1000) == BAD                 # too small
    assert chk(dx=DY) == OK and chk(dx=X) == OK      # in place over dy or x
    assert chk(dx=DY + 4) == BAD                     # partial overlap
    assert chk(dx=DY, lddx=1024, lddy=768) == BAD    # same pointer, other stride
    assert chk(dparams0=DB) == BAD                   # dgamma == dbeta
    assert chk(dparams0=G) == BAD                    # dgamma over gamma
    assert chk(dparams1=WS + 64) == BAD              # dbeta inside the workspace
    assert chk(ws=DX) == BAD                         # workspace over dx
    assert chk(mean=DX) == BAD                       # dx over mean
    assert chk(lddy=700) == BAD and chk(ldx=1024, lddy=800, lddx=768) == OK
    assert chk(dtype=mn.MI_NORM_BF16, x=X + 2) == OK and chk(dtype=mn.MI_NORM_F32, x=X + 2) == BAD
    assert chk(rows=0) == OK
    assert L.mi_norm_bwd_check(None) == BAD
    # the named calls validate the same way (nothing launched on refusal)
    assert L.mi_layernorm_bwd(DY, X, G, MEAN, RSTD, DX, DG, DB, 64, 768, None, 0, None) == BAD
    assert L.mi_rmsnorm_bwd(DY, X, G, RSTD, DY + 4, DG, 64, 768, WS, 1 << 30, None) == BAD


def test_bwd_dispatch(L):
    name = lambda **kw: mn.mi_norm_variant_name(mn.mi_norm_bwd_select(_bprob(**kw)))
    assert name(rows=4096, d=768) == "lnbwd_4_w1_q3_b8"
    assert name(rows=32768, d=8192) == "lnbwd_4_w8_q4_b8"
    # rows of several waves: the fewest of 2 and 4 waves with at most three
    # float32 slots or two 16-bit ones, else 8 waves
    assert name(rows=4096, d=1024) == "lnbwd_4_w1_q4_b8"
    assert name(rows=4096, d=1536) == "lnbwd_4_w2_q3_b8"
    assert name(rows=65536, d=2048) == "lnbwd_4_w4_q2_b8"
    assert name(rows=4096, d=3072) == "lnbwd_4_w4_q3_b8"
    assert name(rows=8192, d=4096) == "lnbwd_4_w8_q2_b8"
    assert name(op=mn.OP_RMSNORM, rows=8192, d=2048) == "rmsbwd_4_w4_q2_b8"
    assert name(op=mn.OP_RMSNORM, rows=2048, d=4096) == "rmsbwd_4_w8_q2_b8"
    assert name(op=mn.OP_RMSNORM, rows=8192, d=8192) == "rmsbwd_4_w8_q4_b8"
    assert name(dtype=mn.MI_NORM_BF16, d=4096) == "lnbwd_bf16_8_w4_q2_b8"
    assert name(op=mn.OP_RMSNORM, d=16384) == "rmsbwd_4_w8_q8_b8"
    assert name(d=16384) == "lnbwd_4_stream_b4_u2"           # past LayerNorm's 24 values per lane
    assert name(dtype=mn.MI_NORM_BF16, d=16384) == "lnbwd_bf16_8_stream_b4_u1"
    assert name(op=mn.OP_RMSNORM, d=32768) == "rmsbwd_4_stream_b4_u2"
    assert name(d=12288) == "lnbwd_4_w8_q6_b8"
    assert name(dtype=mn.MI_NORM_BF16, d=8192) == "lnbwd_bf16_8_w8_q2_b8"
    assert name(dtype=mn.MI_NORM_BF16, d=768) == "lnbwd_bf16_8_w1_q2_b8"
    assert name(dtype=mn.MI_NORM_BF16, op=mn.OP_RMSNORM, d=2048) == "rmsbwd_bf16_8_w1_q4_b8"
    assert name(dtype=mn.MI_NORM_BF16, d=2048) == "lnbwd_bf16_8_w2_q2_b8"
    assert name(dtype=mn.MI_NORM_BF16, d=3072) == "lnbwd_bf16_8_w4_q2_b8"
    assert name(dtype=mn.MI_NORM_BF16, d=6144) == "lnbwd_bf16_8_w8_q2_b8"
    assert name(dtype=mn.MI_NORM_BF16, op=mn.OP_RMSNORM, d=4096) == "rmsbwd_bf16_8_w4_q2_b8"
    assert name(dtype=mn.MI_NORM_BF16, op=mn.OP_RMSNORM, d=8192) == "rmsbwd_bf16_8_w8_q2_b8"
    assert name(d=767) == "lnbwd_1_w2_q8_b8"                  # scalar: 767 elements over 2 waves
    assert name(x=X + 4) == "lnbwd_1_w2_q8_b8"
    assert name(d=9000, x=X + 4) == "lnbwd_1_stream_b4_u8"
    assert name(d=1) == "lnbwd_1_w1_q1_b8"


@pytest.mark.parametrize("op", [mn.OP_LAYERNORM, mn.OP_RMSNORM])
@pytest.mark.parametrize("dt", DTYPES)
def test_bwd_dispatch_covers_every_width(L, op, dt):
    for layout in ("aligned", "misaligned"):
        for d in WIDTHS:
            x = X if layout == "aligned" else X + ESIZE[dt]
            p = _bprob(op=op, rows=4096, d=d, dtype=dt, x=x)
            vid = mn.mi_norm_bwd_select(p)
            assert vid >= 0, (op, dt, d, layout)
            v = mn.mi_norm_variant_get_info(vid)
            assert v["dtype"] == dt and v["op"] == (4 if op == mn.OP_LAYERNORM else 5)
            assert mn.mi_norm_bwd_eligible(vid, p)
            assert v["looped"] or v["max_d"] >= d
            if layout == "aligned" and d % (16 // ESIZE[dt]) == 0 and d <= 12288:
                assert v["vec"] > 1, (d, mn.mi_norm_variant_name(vid))
            if layout == "misaligned":
                assert v["vec"] == 1
    # forward variants are not backward ones, and the reverse
    p = _bprob()
    assert not mn.mi_norm_bwd_eligible(mn.mi_norm_select(_prob(0, 64, 768)), p)
    assert mn.mi_norm_eligible(mn.mi_norm_bwd_select(p), _prob(0, 64, 768)) is False
