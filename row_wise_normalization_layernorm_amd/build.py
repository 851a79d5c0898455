"""Build libmi_norm.so in-tree for gfx950.

Two steps:

1. ``hipcc -c`` compiles, in parallel, the host-side dispatchers, launchers
   and C ABI (csrc/mi_norm.hip forward, csrc/mi_norm_bwd.hip backward) and one
   variant table per row storage type and direction
   (csrc/variants_*.hip, csrc/bwd_variants_*.hip: the gfx950 device code)
   into objects.
2. ``g++ -shared`` links them against the HIP runtime that PyTorch ships.

The link step matters: torch's ``libamdhip64.so`` carries no SONAME and is
loaded under that bare name, while /opt/rocm's copy has SONAME
``libamdhip64.so.7``.  Linking against /opt/rocm's copy would make the loader
map a second HIP runtime beside torch's, and torch's streams would mean
nothing to it.  Linking against torch's copy records ``NEEDED
libamdhip64.so``, which the loader resolves to the runtime torch already has
in the process.  The run path lists torch's lib directory first and
/opt/rocm/lib second, so the library also loads without torch.
"""
from __future__ import annotations

import importlib.util
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmi_norm.so")
BENCH_LIB = os.path.join(PKG, "libmi_norm_bench.so")
SOURCES = ("mi_norm.hip", "variants_f32.hip", "variants_f16.hip", "variants_bf16.hip",
           "mi_norm_bwd.hip", "bwd_variants_f32.hip", "bwd_variants_f16.hip", "bwd_variants_bf16.hip")
HEADERS = ("norm_kernels.hpp", "variant_table.hpp", "host_common.hpp", "bwd_kernels.hpp", "bwd_table.hpp")
BENCH_SOURCES = ("bench_loop.cpp",)
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    # keep hipcc from forming packed-FP32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def rocm_path() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def torch_lib_dir() -> str:
    spec = importlib.util.find_spec("torch")
    if spec is None or spec.origin is None:
        raise RuntimeError("PyTorch is not importable; its HIP runtime is the one to link")
    d = os.path.join(os.path.dirname(spec.origin), "lib")
    if not os.path.exists(os.path.join(d, "libamdhip64.so")):
        raise RuntimeError(f"no libamdhip64.so under {d}")
    return d


def source_paths() -> list[str]:
    return [os.path.join(CSRC, s) for s in SOURCES + HEADERS] + [os.path.join(INCLUDE, h) for h in ("mi_norm.h", "mi_norm_tuning.h")]


def _run(cmd: list[str], verbose: bool, stderr_to: str | None = None) -> None:
    _wait(_start(cmd, verbose, stderr_to))


def _start(cmd: list[str], verbose: bool, stderr_to: str | None = None):
    if verbose:
        print(" ".join(cmd), flush=True)
    f = open(stderr_to, "w") if stderr_to else None
    return cmd, subprocess.Popen(cmd, stderr=f), f, stderr_to


def _wait(job) -> None:
    cmd, proc, f, stderr_to = job
    rc = proc.wait()
    if f:
        f.close()
    if rc != 0:
        if stderr_to:
            with open(stderr_to) as f:
                sys.stderr.write("".join(l for l in f if "remark:" not in l))
        raise subprocess.CalledProcessError(rc, cmd)


def build(verbose: bool = False, resource_report: bool = True, full_table: bool | None = None) -> str:
    """Compile and link libmi_norm.so; returns its path.

    With ``resource_report`` the compiler's per-kernel resource remarks
    (VGPRs, SGPRs, LDS, occupancy) are written to _build/resource_usage.txt.
    ``full_table`` (default: the environment variable MI_NORM_FULL_TABLE set
    to 1) compiles every (waves per row, slots, workgroup) variant instead of
    the ones the dispatcher can choose, for sweeps that force variants.
    """
    if full_table is None:
        full_table = os.environ.get("MI_NORM_FULL_TABLE") == "1"
    hipcc = os.path.join(rocm_path(), "bin", "hipcc")
    if not os.path.exists(hipcc):
        hipcc = shutil.which("hipcc") or hipcc
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs, jobs, reports = [], [], []
    for src in SOURCES:
        stem = os.path.splitext(src)[0]
        obj = os.path.join(BUILD_DIR, stem + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, *(["-DMI_NORM_FULL_TABLE"] if full_table else []), "-I", INCLUDE, "-I", CSRC,
               "-c", os.path.join(CSRC, src), "-o", obj]
        report = os.path.join(BUILD_DIR, f"remarks_{stem}.txt")
        if resource_report:
            cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
            reports.append(report)
        jobs.append(_start(cmd, verbose, stderr_to=report))
        objs.append(obj)
    failed = None
    for job in jobs:
        try:
            _wait(job)
        except subprocess.CalledProcessError as e:
            failed = failed or e
    if failed:
        raise failed
    if resource_report:
        with open(os.path.join(BUILD_DIR, "resource_usage.txt"), "w") as out:
            for r in reports:
                with open(r) as f:
                    out.write(f.read())
    tlib = torch_lib_dir()
    rlib = os.path.join(rocm_path(), "lib")
    tmp = LIB + ".tmp"
    cmd = ["g++", "-shared", "-Wl,-soname,libmi_norm.so", "-o", tmp, *objs, f"-L{tlib}", "-l:libamdhip64.so",
           f"-Wl,-rpath,{tlib}:{rlib}", "-Wl,--no-undefined", "-Wl,--no-as-needed"]
    _run(cmd, verbose)
    os.replace(tmp, LIB)
    build_bench(verbose)
    return LIB


def build_bench(verbose: bool = False) -> str:
    """Host-only timing loops used by bench.py, linked to libmi_norm.so."""
    tmp = BENCH_LIB + ".tmp"
    cmd = ["g++", "-O2", "-fPIC", "-shared", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", os.path.join(rocm_path(), "include"),
           *[os.path.join(CSRC, s) for s in BENCH_SOURCES], "-o", tmp,
           f"-L{PKG}", "-l:libmi_norm.so", "-Wl,-rpath,$ORIGIN", "-Wl,--no-undefined",
           f"-L{torch_lib_dir()}", "-l:libamdhip64.so"]
    _run(cmd, verbose)
    os.replace(tmp, BENCH_LIB)
    return BENCH_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
