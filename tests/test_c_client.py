"""The C ABI from plain C: tests/c_client/client.c includes only
include/mi_norm.h, include/mi_norm_tuning.h (and HIP's C runtime header), links libmi_norm.so, and is
compiled here with gcc -std=c99 -Werror.  On the CPU its struct layouts and
the host-only calls must agree with the Python binding; on the GPU it runs
LayerNorm (named call) and bfloat16 fused add + RMSNorm (general call) and
its outputs are checked against the float64 oracle."""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import row_wise_normalization_layernorm_amd as mn
from row_wise_normalization_layernorm_amd import _binding as B
from row_wise_normalization_layernorm_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_client", "client.c")


@pytest.fixture(scope="module")
def client(tmp_path_factory):
    import torch
    mn.lib()  # the library must be built
    pkg = os.path.dirname(B.LIB_PATH)
    tlib = os.path.join(os.path.dirname(torch.__file__), "lib")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = str(tmp_path_factory.mktemp("c_client") / "client")
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"), SRC, "-o", exe,
           f"-L{pkg}", "-l:libmi_norm.so", f"-L{tlib}", "-l:libamdhip64.so", f"-Wl,-rpath,{pkg}:{tlib}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, *args, timeout=120):
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    return r.stdout


def test_struct_layouts_match_the_binding(client):
    out = _run(client, "layout")
    sizes, offsets = {}, {}
    for line in out.splitlines():
        name, val = line.split()
        (offsets if "." in name else sizes)[name] = int(val)
    for cname, cls in (("mi_norm_problem", B.Problem), ("mi_norm_bwd_problem", B.BwdProblem),
                       ("mi_norm_variant_info", B.VariantInfo)):
        assert sizes[cname] == ctypes.sizeof(cls), cname
        fields = [f for f, _ in cls._fields_]
        assert sorted(fields) == sorted(k.split(".", 1)[1] for k in offsets if k.startswith(cname + ".")), cname
        for f in fields:
            assert offsets[f"{cname}.{f}"] == getattr(cls, f).offset, (cname, f)


def test_host_calls_agree_with_the_binding(client):
    got = dict(line.split(" ", 1) for line in _run(client, "host").splitlines())
    assert got["version"] == mn.mi_norm_version()
    assert got["check_ln"] == "0" and got["check_bad"] == "1"
    fake = lambda n: n << 36
    p = mn.problem(mn.OP_LAYERNORM, 4096, 768, fake(1), fake(2), fake(3), fake(4))
    vid = mn.mi_norm_select(p)
    assert got["select_ln"] == mn.mi_norm_variant_name(vid)
    v = mn.mi_norm_variant_get_info(vid)
    assert got["info_ln"] == f"0 {v['waves_per_row']} {v['slots']} {v['waves_per_block']} {v['rows_per_lane']}"
    big = mn.problem(mn.OP_LAYERNORM, 32768, 8192, fake(1), fake(2), fake(3), fake(4))
    assert got["select_big"] == mn.mi_norm_variant_name(mn.mi_norm_select(big))
    assert got["status"] == mn.mi_norm_status_string(mn.MI_NORM_ERR_INVALID)
    b = mn.bwd_problem(mn.OP_LAYERNORM, 4096, 768, fake(5), fake(6), fake(7), fake(8), fake(9), fake(10),
                       fake(11), fake(12), None, 0)
    assert int(got["bwd_workspace"]) == mn.mi_norm_bwd_workspace_size(b)
    assert int(got["variants"]) == mn.mi_norm_variant_count()


@pytest.mark.gpu
def test_c_caller_on_the_gpu(client, tmp_path):
    rows, d = 1031, 1000
    print(f"C client run [{rows}x{d}]", flush=True)
    x = wl.make_x(rows, d, "offset", [31, rows, d])
    g, bta = wl.make_affine(d, [31, d])
    xb = wl.make_x16(rows, d, "normal", [32, rows, d], wl.BF16)
    rb = wl.make_x16(rows, d, "normal", [33, rows, d], wl.BF16)
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        for a in (x, g, bta, xb, rb):
            f.write(np.ascontiguousarray(a).tobytes())
    assert _run(client, "run", str(inp), str(outp), str(rows), str(d)).strip() == "ok"
    raw = np.fromfile(outp, dtype=np.uint8)
    n = rows * d
    off = 0

    def take(count, dtype):
        nonlocal off
        a = raw[off:off + count * np.dtype(dtype).itemsize].view(dtype)
        off += count * np.dtype(dtype).itemsize
        return a

    y, mean, rstd = take(n, np.float32), take(rows, np.float32), take(rows, np.float32)
    yb, hb, rstdb = take(n, np.uint16), take(n, np.uint16), take(rows, np.float32)
    assert off == raw.size
    ry, rm, rr, _, _ = oracle.layernorm(x, g, bta, wl.EPS)
    for got, want, what in ((y, ry.reshape(-1), "y"), (mean, rm, "mean"), (rstd, rr, "rstd")):
        ok, err, ratio = oracle.tolerance_ok(got, want)
        assert ok, f"{what}: max abs err {err:.3e}, err/bound {ratio:.3f}"
    _, y64, h, s = oracle.add_rmsnorm16(xb, rb, oracle.FMT_BF16, g, wl.EPS)
    ok, err, ratio = oracle.tolerance_ok16(yb.reshape(rows, d), y64, oracle.FMT_BF16)
    assert ok, f"bf16 y: max abs err {err:.3e}, err/bound {ratio:.3f}"
    assert np.array_equal(hb.reshape(rows, d), h.view(np.uint16)), "h != x + r"
    assert oracle.tolerance_ok(rstdb, s)[0]
