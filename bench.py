#!/usr/bin/env python3
"""Benchmark: forward LayerNorm FP32 [4096,768] with per-row mean/rstd on one MI355X.

One step is one call of the C ABI (mi_layernorm_fwd: validation, dispatch and
one kernel launch) over one batch of seeded synthetic input already resident
in HBM.  The run:

1. draws the inputs (row_wise_normalization_layernorm_amd.workloads) and
   copies them to the device;
2. checks the GPU output against the float64 oracle and refuses to time on a
   mismatch (correctness gates timing);
3. runs W untimed warm-up steps, then times exactly K steps between HIP events
   recorded on the stream the kernels run on, with a device synchronization
   on both sides;
4. times the oracle on the host cores as a reported CPU baseline;
5. prints one JSON line.

HBM, not cache: in the default "rotate" mode, step s reads buffer set
s % n_sets, with enough sets that their total footprint is at least 1 GiB
(four times the 256 MB Infinity Cache); "warm" reuses one set, as the pages'
own timers did, and measures cache-resident bandwidth.

Algorithmic bytes per step (LayerNorm): read x and write y (8 B per element),
read gamma and beta (8 B per column), write mean and rstd (8 B per row).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time
from typing import NamedTuple

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published peak
METRIC = "achieved HBM GB/s (% of peak) + kernel µs, LayerNorm FP32 [4096,768]"

class W(NamedTuple):
    """A benchmark workload: operation, row storage type, shape, input
    pattern, whether per-row statistics are written, and the extra elements
    in each row's stride (0: contiguous rows)."""
    op: str
    storage: str
    rows: int
    d: int
    pattern: str = "normal"
    stats: bool = False
    pad: int = 0


BENCH_WORKLOADS = {
    "ln_4096x768": W("layernorm", "f32", 4096, 768, "normal", True),
    "ln_512x128": W("layernorm", "f32", 512, 128),
    "ln_8192x768": W("layernorm", "f32", 8192, 768, "offset"),
    "ln_1024x2048": W("layernorm", "f32", 1024, 2048, "offset"),
    "ln_4096x4096": W("layernorm", "f32", 4096, 4096, "offset"),
    "ln_32768x8192": W("layernorm", "f32", 32768, 8192),
    # one GPU's share when the rows of [4096,768] and [32768,8192] are split over eight
    "ln_512x768": W("layernorm", "f32", 512, 768, "normal", True),
    "ln_4096x8192": W("layernorm", "f32", 4096, 8192),
    "rms_512x128": W("rmsnorm", "f32", 512, 128),
    "rms_4096x768": W("rmsnorm", "f32", 4096, 768),
    "rms_2048x4096": W("rmsnorm", "f32", 2048, 4096),
    "rms_8192x8192": W("rmsnorm", "f32", 8192, 8192),
    "rms_256x8193": W("rmsnorm", "f32", 256, 8193),
    "addln_4096x768": W("add_layernorm", "f32", 4096, 768, "normal", True),
    "addln_32768x8192": W("add_layernorm", "f32", 32768, 8192),
    "addrms_4096x768": W("add_rmsnorm", "f32", 4096, 768),
    "addrms_2048x4096": W("add_rmsnorm", "f32", 2048, 4096),
    # 16-bit row storage, float32 statistics and arithmetic
    "ln_bf16_4096x768": W("layernorm", "bf16", 4096, 768, "normal", True),
    "ln_f16_4096x768": W("layernorm", "f16", 4096, 768, "normal", True),
    "ln_bf16_32768x8192": W("layernorm", "bf16", 32768, 8192),
    "ln_f16_32768x8192": W("layernorm", "f16", 32768, 8192),
    "rms_bf16_2048x4096": W("rmsnorm", "bf16", 2048, 4096),
    "rms_bf16_8192x8192": W("rmsnorm", "bf16", 8192, 8192),
    "addrms_bf16_4096x768": W("add_rmsnorm", "bf16", 4096, 768),
    "addln_bf16_32768x8192": W("add_layernorm", "bf16", 32768, 8192),
    # backward (dx and the parameter gradients) from the forward's statistics
    "lnbwd_4096x768": W("layernorm_bwd", "f32", 4096, 768),
    "lnbwd_32768x8192": W("layernorm_bwd", "f32", 32768, 8192),
    "rmsbwd_4096x768": W("rmsnorm_bwd", "f32", 4096, 768),
    "rmsbwd_8192x8192": W("rmsnorm_bwd", "f32", 8192, 8192),
    "lnbwd_bf16_4096x768": W("layernorm_bwd", "bf16", 4096, 768),
    "lnbwd_bf16_32768x8192": W("layernorm_bwd", "bf16", 32768, 8192),
    # strided rows: each row of x and y sits in a wider row of its buffer
    "ln_4096x768_ld1024": W("layernorm", "f32", 4096, 768, "normal", True, 256),
    "ln_bf16_32768x8192_ld8448": W("layernorm", "bf16", 32768, 8192, "normal", False, 256),
    # calibration copies: float32 elements moving the same bytes as a shape
    "copy_4096x768": W("copy", "f32", 4096, 768),
    "copy_32768x8192": W("copy", "f32", 32768, 8192),
    "copy_4096x384": W("copy", "f32", 4096, 384),      # the bytes of a 16-bit [4096,768]
    "copy_16384x8192": W("copy", "f32", 16384, 8192),  # the bytes of a 16-bit [32768,8192]
    "copy_4096x4096": W("copy", "f32", 4096, 4096),
    # the parts of a launch: an empty kernel, and passes that only read or
    # only write the bytes of x (or y) of [4096,768]
    "empty": W("empty", "f32", 0, 0),
    "read_4096x768": W("read", "f32", 4096, 768),
    "write_4096x768": W("write", "f32", 4096, 768),
}

ESIZE = {"f32": 4, "f16": 2, "bf16": 2}

# the device code of the kernels and the tables that instantiate them (launch
# shapes included), per direction; a profile's counters stand for the kernels
# only while these are unchanged and the dispatcher still picks the profiled
# variant
_CSRC = "row_wise_normalization_layernorm_amd/csrc/"
KERNEL_SOURCES = {
    "fwd": tuple(_CSRC + f for f in ("norm_kernels.hpp", "variant_table.hpp", "variants_f32.hip",
                                     "variants_f16.hip", "variants_bf16.hip")),
    "bwd": tuple(_CSRC + f for f in ("norm_kernels.hpp", "bwd_kernels.hpp", "bwd_table.hpp",
                                     "bwd_variants_f32.hip", "bwd_variants_f16.hip", "bwd_variants_bf16.hip")),
}


_CODE_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/|\s+|[^"\'/\s]+|/',
                          re.S)


def code_text(src: str) -> str:
    """The source with its comments dropped and each run of white space made
    one blank: what the compiler sees, so that rewording a comment leaves the
    pairing of the committed counter summaries intact."""
    out = []
    for tok in _CODE_TOKENS.findall(src):
        if tok.startswith("//") or tok.startswith("/*") or tok.isspace():
            if out and out[-1] != " ":
                out.append(" ")
        else:
            out.append(tok)
    return "".join(out).strip()


def kernel_source_hash(direction: str = "fwd") -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[direction]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def direction_of(workload: str) -> str:
    return "bwd" if BENCH_WORKLOADS[workload].op.endswith("_bwd") else "fwd"


def algorithmic_bytes(op: str, rows: int, d: int, stats: bool, storage: str = "f32") -> int:
    """Bytes a step must move: x read and y written (one element each); the
    fused ops also read r and write h = x + r; gamma/beta (or w, float32)
    once; the per-row float32 statistics when requested.  The backward reads
    dy and x, writes dx, reads gamma (w) and the statistics and writes the
    parameter gradients; its workspace traffic is overhead, not counted.  Row
    padding is not touched and does not count."""
    e = ESIZE[storage]
    if op.endswith("_bwd"):
        ln = op.startswith("layernorm")
        return 3 * e * rows * d + (12 if ln else 8) * d + (8 if ln else 4) * rows
    if op in ("read", "write"):
        return 4 * rows * d
    if op == "empty":
        return 0
    per_elem = (4 if op.startswith("add_") else 2) * e
    if op.endswith("layernorm"):
        return per_elem * rows * d + 8 * d + (8 * rows if stats else 0)
    if op.endswith("rmsnorm"):
        return per_elem * rows * d + 4 * d + (4 * rows if stats else 0)
    return 8 * rows * d  # copy: one float32 read, one written per element


def describe(op: str, rows: int, d: int, stats: bool, storage: str = "f32", pad: int = 0) -> str:
    if op == "copy":
        return f"streaming copy FP32 {rows*d} elements (calibration, bytes of [{rows},{d}])"
    if op == "empty":
        return "empty kernel, 256 workgroups of 1024 threads (calibration)"
    if op in ("read", "write"):
        return f"{op}-only pass over {rows*d} FP32 elements (calibration, the bytes of x of [{rows},{d}])"
    kind = {"f32": "FP32", "f16": "FP16 storage, FP32 statistics",
            "bf16": "BF16 storage, FP32 statistics"}[storage]
    if op.endswith("_bwd"):
        grads = "dx, dgamma, dbeta" if op.startswith("layernorm") else "dx, dw"
        name = "LayerNorm" if op.startswith("layernorm") else "RMSNorm"
        return f"{name} backward ({grads}) {kind} [{rows},{d}]"
    name = "LayerNorm" if op.endswith("layernorm") else "RMSNorm"
    if op.startswith("add_"):
        name = "residual add (h = x + r written) + " + name
    ln = op.endswith("layernorm")
    extra = " with per-row mean/rstd" if (stats and ln) else (" with rstd" if stats else "")
    kind = {"f32": "FP32", "f16": "FP16 storage, FP32 statistics",
            "bf16": "BF16 storage, FP32 statistics"}[storage]
    strided = f", rows at stride {d + pad}" if pad else ""
    return f"{name} fwd {kind} [{rows},{d}]{extra}{strided}"


def pmc_traffic(workload: str, variant: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none, the kernels changed since it was taken, or the run uses
    another variant than the one profiled."""
    path = os.path.join(ROOT, "profiles", f"{workload}.txt")
    if not os.path.exists(path):
        return None, None
    text = open(path).read()
    m = re.search(r"^kernel_source_sha256:\s*(\w+)", text, re.M)
    t = re.search(r"^traffic_bytes_per_launch:\s*([\d.eE+]+)", text, re.M)
    v = re.search(r"^kernel_variant:\s*(\S+)", text, re.M)
    if not m or not t or not v or m.group(1) != kernel_source_hash(direction_of(workload)) or v.group(1) != variant:
        return None, path
    return float(t.group(1)), path


def trace_stats(workload: str, variant: str):
    """Per-dispatch kernel durations (µs: median, min, max, mean over the
    timed steps) from the committed rocprofv3 kernel-trace summary, or None
    when there is none, the kernels changed since it was taken, or the run
    uses another variant than the one traced."""
    path = os.path.join(ROOT, "profiles", f"{workload}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    field = lambda k: (re.search(rf"^{k}:\s*(\S+)", text, re.M) or [None, None])[1]
    if field("kernel_source_sha256") != kernel_source_hash(direction_of(workload)) or field("kernel_variant") != variant:
        return None
    try:
        out = {k: float(field(f"dispatch_us_{k}")) for k in ("median", "min", "max", "mean")}
        out["dispatches"] = int(field("dispatches"))
    except (TypeError, ValueError):
        return None
    out["source"] = os.path.relpath(path, ROOT)
    out["what"] = ("rocprofv3 --kernel-trace, per-dispatch durations of the timed steps; the tracer runs "
                   "each dispatch longer than an untraced back-to-back one (the summary gives both)")
    u = field("untraced_span_us_per_step")
    out["untraced_span_us_of_that_run"] = float(u) if u else None
    return out


def load_bench_lib():
    import row_wise_normalization_layernorm_amd as mn
    mn.lib()
    from row_wise_normalization_layernorm_amd import build as B
    if not os.path.exists(B.BENCH_LIB):
        raise RuntimeError(f"{B.BENCH_LIB} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(B.BENCH_LIB)
    P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    L.mi_bench_layernorm_loop.argtypes = [P, P, P, P, P, P, I, I64, I64, F, I, I, P]
    L.mi_bench_rmsnorm_loop.argtypes = [P, P, P, P, I, I64, I64, F, I, I, P]
    L.mi_bench_add_layernorm_loop.argtypes = [P, P, P, P, P, P, P, P, I, I64, I64, F, I, I, P]
    L.mi_bench_add_rmsnorm_loop.argtypes = [P, P, P, P, P, P, I, I64, I64, F, I, I, P]
    L.mi_bench_copy_loop.argtypes = [P, P, I, I64, I, P]
    L.mi_bench_norm_loop.argtypes = [P, P, P, P, P, P, P, I, I, I, P]
    L.mi_bench_bwd_loop.argtypes = [P, P, P, P, P, P, P, P, I, I, I, P]
    L.mi_bench_calib_loop.argtypes = [I, P, P, I, I64, I, P]
    return L


def ptr_array(tensors):
    return (ctypes.c_void_p * len(tensors))(*[t.data_ptr() if t is not None else None for t in tensors])


def oracle_call(op, x, r, params, eps, storage: str = "f32"):
    """(y, h, [stats...]) from the oracle for one input batch; for 16-bit
    storage y is the float64 output before its rounding (what the 16-bit
    acceptance bound is measured from) and x, r, h are bit patterns."""
    import oracle
    if storage != "f32":
        f = oracle.FMT_F16 if storage == "f16" else oracle.FMT_BF16
        if op == "layernorm":
            _, y64, mean, rstd = oracle.layernorm16(x, f, *params, eps)
            return y64, None, [mean, rstd]
        if op == "rmsnorm":
            _, y64, rstd = oracle.rmsnorm16(x, f, *params, eps)
            return y64, None, [rstd]
        if op == "add_layernorm":
            _, y64, h, mean, rstd = oracle.add_layernorm16(x, r, f, *params, eps)
            return y64, h, [mean, rstd]
        _, y64, h, rstd = oracle.add_rmsnorm16(x, r, f, *params, eps)
        return y64, h, [rstd]
    if op == "layernorm":
        y, mean, rstd, _, _ = oracle.layernorm(x, *params, eps)
        return y, None, [mean, rstd]
    if op == "rmsnorm":
        y, rstd, _ = oracle.rmsnorm(x, *params, eps)
        return y, None, [rstd]
    if op == "add_layernorm":
        y, h, mean, rstd = oracle.add_layernorm(x, r, *params, eps)
        return y, h, [mean, rstd]
    y, h, rstd = oracle.add_rmsnorm(x, r, *params, eps)
    return y, h, [rstd]


def time_oracle(call, budget_s: float, threads: int | None = None):
    """Repeat ``call`` (one oracle pass over the workload) until ``budget_s``
    of wall time has passed, on ``threads`` OpenMP threads (None: all the
    host gives); returns (repetitions, seconds, threads used)."""
    import oracle
    most = oracle.max_threads()
    n = most if threads is None else min(threads, most)
    oracle.set_threads(n)
    try:
        call()  # the first call loads the library and touches the pages
        reps, t0 = 0, time.perf_counter()
        while True:
            call()
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                return reps, el, n
    finally:
        oracle.set_threads(most)


def cpu_baseline(op, x, r, params, eps, budget_s: float, storage: str = "f32", threads: int | None = None):
    """The float64 oracle on the host cores over the same workload."""
    return time_oracle(lambda: oracle_call(op, x, r, params, eps, storage), budget_s, threads)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def gate_cycles(steps: int) -> int:
    """Spin-kernel length (shader clock cycles at 2.4 GHz) that holds a stream
    for about 5 us per step to be queued behind it, 80 us to 2 ms."""
    return int(2400 * min(2000.0, max(80.0, 5.0 * steps)))


def gated_span(torch, stream, steps: int, enqueue, tries: int = 4):
    """Time ``enqueue()``, which queues ``steps`` launches on ``stream``,
    between two stream events behind a spin kernel.

    A spin kernel ahead of the start event holds the stream while the host
    enqueues the launches, so the span between the events holds GPU time
    only.  Without it the idle GPU records the start event at once and then
    waits for the host's first launch; and a host call costs 3-4 us, close
    to a small kernel's time, so a host stall could leave the GPU idle
    inside the span.  The gate worked if the start event was still pending
    once the last launch was queued; if it had already completed, the run
    is repeated behind a spin twice as long (at most ``tries`` runs).
    Returns (ms of the span, wall ms of the last run, gate us, covered)."""
    cycles = gate_cycles(steps)
    for attempt in range(tries):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        with torch.cuda.stream(stream):
            torch.cuda._sleep(cycles)
        t0.record(stream)
        enqueue()
        covered = not t0.query()
        t1.record(stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - w0) * 1e3
        if covered or attempt == tries - 1:
            break
        cycles *= 2
    return t0.elapsed_time(t1), wall_ms, cycles / 2400, covered


def copy_reference(torch, BL, stream, bytes_step: int, steps: int, warmup: int, mode: str,
                   footprint_gib: float):
    """The calibration copy moving a step's bytes (half read, half written),
    timed like the step on rotated buffers: (µs per copy, buffer sets)."""
    n = max(4, (bytes_step // 8) // 4 * 4)
    nsets = 1 if mode == "warm" else max(1, math.ceil(footprint_gib * 2**30 / (8 * n)))
    dev = torch.device("cuda:0")
    srcs = [torch.zeros(n, device=dev) for _ in range(nsets)]
    dsts = [torch.empty(n, device=dev) for _ in range(nsets)]
    torch.cuda.synchronize()
    sa, da = ptr_array(srcs), ptr_array(dsts)
    sh = stream.cuda_stream
    if BL.mi_bench_copy_loop(sa, da, nsets, n, warmup, sh) != 0:
        raise RuntimeError("copy loop failed")
    torch.cuda.synchronize()

    def enqueue():
        if BL.mi_bench_copy_loop(sa, da, nsets, n, steps, sh) != 0:
            raise RuntimeError("copy loop failed")

    ms, _, _, _ = gated_span(torch, stream, steps, enqueue)   # the same gate as the timed steps
    us = ms * 1e3 / steps
    del srcs, dsts
    return us, nsets


def measure_and_print(args, torch, stream, run_native, run_python, rotated, nsets, per_set, variant_name,
                      bytes_step, parity, cpu_fn, workload, config, rows) -> int:
    """Warm-up, the timed steps between stream events, the single launches,
    and the one JSON line.  ``run_native(k[, arrays])`` / ``run_python(k,
    start)`` run k steps; ``rotated(first)`` gives the pointer arrays from
    buffer set ``first``; ``cpu_fn(budget)`` times the oracle."""
    # -- warm-up and timed steps
    if args.launch == "graph":
        gw, graph = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw, stream=stream):
            run_python(args.warmup)
        with torch.cuda.graph(graph, stream=stream):
            run_python(args.steps, start=args.warmup)
        runner_w, runner_t = gw.replay, graph.replay
    elif args.launch == "native":
        runner_w, runner_t = (lambda: run_native(args.warmup)), (lambda: run_native(args.steps))
    else:
        def runner_w():
            run_python(args.warmup)

        def runner_t():
            run_python(args.steps, start=args.warmup)

    with torch.cuda.stream(stream):
        runner_w()
    torch.cuda.synchronize()

    def enqueue():
        with torch.cuda.stream(stream):
            runner_t()

    ms, wall_ms, gate_us, covered = gated_span(torch, stream, args.steps, enqueue,
                                               tries=1 if args.profile else 4)
    ms_per_step = ms / args.steps

    # single launches on an idle GPU, each between two events: the duration a
    # kernel tracer reports per dispatch (no overlap with a neighbour's drain).
    # A short spin kernel holds the stream while the host enqueues the first
    # event and the launch, so the span holds no host time.
    iso = []
    if args.launch == "native" and not args.profile:
        for i in range(20):
            arrays = rotated((args.steps + i) % nsets)   # a set last touched about n_sets steps ago
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                torch.cuda._sleep(200000)
                e0.record(stream)
                run_native(1, arrays)
                e1.record(stream)
            torch.cuda.synchronize()
            iso.append(e0.elapsed_time(e1) * 1e3)
    iso_us = round(sorted(iso)[len(iso) // 2], 3) if iso else None
    gbps = bytes_step / (ms_per_step * 1e-3) / 1e9

    traffic, _ = pmc_traffic(args.workload, variant_name)
    dispatch = trace_stats(args.workload, variant_name)
    roofline = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(gbps / PEAK_HBM_GBPS, 4),
                "traffic": traffic, "kernel": variant_name,
                "algorithmic_bytes_per_launch": bytes_step,
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-scaled)"}

    copy = None
    calib = BENCH_WORKLOADS[args.workload].op in ("copy", "empty", "read", "write")
    if not args.no_copy and not args.profile and args.launch == "native" and not calib:
        copy_us, copy_sets = copy_reference(torch, load_bench_lib(), stream, bytes_step, args.steps,
                                            args.warmup, args.mode, args.footprint_gib)
        copy = {"us": round(copy_us, 3), "bytes": 8 * max(4, (bytes_step // 8) // 4 * 4),
                "buffer_sets": copy_sets,
                "pct_of_copy": round(100 * copy_us / (ms_per_step * 1e3), 2),
                "what": "copy_cover moving the step's bytes (half read, half written), timed the same way"}

    cpu = None
    if cpu_fn is not None and not args.profile:
        reps, el, threads = cpu_fn(args.cpu_seconds, None)
        reps1, el1, _ = cpu_fn(args.cpu_seconds / 2, 1)
        cpu = {"value": round(bytes_step * reps / el / 1e9, 3), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"full {workload} workload, {reps} repetitions "
                         f"({el:.2f} s wall, float64 C oracle, OpenMP over rows)",
               "value_1core": round(bytes_step * reps1 / el1 / 1e9, 3),
               "sample_1core": f"{reps1} repetitions ({el1:.2f} s wall) on one thread",
               "ms_per_pass": round(el * 1e3 / reps, 3),
               "cpu_model": cpu_model()}

    line = {
        "metric": (METRIC if args.workload == "ln_4096x768" else f"achieved HBM GB/s, {workload}"),
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": config.get("storage", "f32"),
        "data": "synthetic",
        "config": {"workload": workload, **config, "mode": args.mode, "buffer_sets": nsets,
                   "footprint_bytes": nsets * per_set, "launch": args.launch, "variant": variant_name,
                   "arithmetic": "f32", "hip_force_dev_kernarg": os.environ.get("HIP_FORCE_DEV_KERNARG"),
                   "parallelism": "single GPU"},
        "span_us_per_step": round(ms_per_step * 1e3, 3),
        "kernel_dispatch_us": dispatch,
        "isolated_launch_us": iso_us,
        "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
        "rows_per_s": round(rows / (ms_per_step * 1e-3), 1),
        "wall_ms_per_step": round(wall_ms / args.steps, 6),
        "gate": {"us": round(gate_us, 1), "covered": covered},
        "parity": parity,
        "roofline": roofline,
        "copy_reference": copy,
        "cpu_baseline": cpu,
        "kernel_source_sha256": kernel_source_hash(direction_of(args.workload)),
        "profile_run": bool(args.profile),
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_bwd(args, torch, np, mn, wl, dev, wk) -> int:
    """Backward workloads: one mi_norm_bwd call per step (the row kernel and
    the column reduction of the parameter gradients), on inputs resident in
    HBM, parity-gated against the float64 oracle."""
    import oracle
    op_b, storage, rows, d, pattern, _, pad = wk
    ln = op_b.startswith("layernorm")
    es, ld = ESIZE[storage], d + pad
    dtcode = {"f32": mn.MI_NORM_F32, "f16": mn.MI_NORM_F16, "bf16": mn.MI_NORM_BF16}[storage]
    tdtype = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[storage]
    eps = wl.EPS
    BL = load_bench_lib()

    seed = wl.case_seed(7, rows, d, pattern)
    x_h = wl.make_x(rows, d, pattern, seed)
    dy_h = wl.make_x(rows, d, "normal", [8] + seed)
    p0_h = wl.make_affine(d, [7, d, 99])[0] if ln else wl.make_weight(d, [7, d, 99])
    fmt = None
    if storage != "f32":
        fmt = wl.F16 if storage == "f16" else wl.BF16
        x_h, dy_h = wl.quantize16(x_h, fmt), wl.quantize16(dy_h, fmt)
        xw = oracle.widen16(x_h, fmt)
    else:
        xw = x_h
    if ln:
        _, mean_h, rstd_h, _, _ = oracle.layernorm(xw, p0_h, np.zeros(d, np.float32), eps)
    else:
        _, rstd_h, _ = oracle.rmsnorm(xw, p0_h, eps)
        mean_h = None

    per_set = 3 * es * rows * ld + 8 * rows
    nsets = 1 if args.mode == "warm" else max(1, math.ceil(args.footprint_gib * 2**30 / per_set))

    def device_rows(host):
        t = torch.from_numpy(host.view(np.int16) if es == 2 else host).to(dev)
        t = t.view(tdtype) if es == 2 else t
        if pad == 0:
            return t
        buf = torch.zeros(rows, ld, dtype=tdtype, device=dev)
        buf[:, :d].copy_(t)
        return buf[:, :d]

    def empty_rows():
        return torch.empty(rows, ld, dtype=tdtype, device=dev)[:, :d]

    xs = [device_rows(x_h) for _ in range(nsets)]
    dys = [device_rows(dy_h) for _ in range(nsets)]
    dxs = [empty_rows() for _ in range(nsets)]
    means = [torch.from_numpy(mean_h).to(dev) for _ in range(nsets)] if ln else None
    rstds = [torch.from_numpy(rstd_h).to(dev) for _ in range(nsets)]
    dgs = [torch.empty(d, device=dev) for _ in range(nsets)]
    dbs = [torch.empty(d, device=dev) for _ in range(nsets)] if ln else None
    p0 = torch.from_numpy(p0_h).to(dev)
    opcode = mn.OP_LAYERNORM if ln else mn.OP_RMSNORM

    def problem_for(j, ws=None, ws_bytes=0):
        return mn.bwd_problem(opcode, rows, d, dys[j], xs[j], dxs[j], p0, means[j] if ln else None, rstds[j],
                              dgs[j], dbs[j] if ln else None, ws, ws_bytes, dtype=dtcode, lddy=ld, ldx=ld, lddx=ld)

    nbytes = mn.mi_norm_bwd_workspace_size(problem_for(0))
    workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    probs = [problem_for(j, workspace, nbytes) for j in range(nsets)]
    torch.cuda.synchronize()

    vid = -1
    if args.variant:
        names = [mn.mi_norm_variant_name(i) for i in range(mn.mi_norm_variant_count())]
        if args.variant not in names:
            print(f"unknown variant {args.variant}", file=sys.stderr)
            return 1
        vid = names.index(args.variant)
    variant_name = mn.mi_norm_variant_name(vid if vid >= 0 else mn.mi_norm_bwd_select(probs[0]))

    stream = torch.cuda.Stream(device=dev)
    sh = stream.cuda_stream

    def rot(ts, first):
        return None if ts is None else ptr_array(ts[first:] + ts[:first])

    def rotated(first: int):
        return tuple(rot(t, first) for t in (dys, xs, dxs, means, rstds, dgs, dbs))

    base_arrays = rotated(0)

    def run_native(k: int, arrays=None):
        a = arrays if arrays is not None else base_arrays
        st = BL.mi_bench_bwd_loop(ctypes.byref(probs[0]), *a, nsets, k, vid, sh)
        if st != 0:
            raise RuntimeError(f"bench loop failed: {mn.mi_norm_status_string(st)}")

    def run_python(k: int, start: int = 0):
        for s_ in range(start, start + k):
            if vid < 0:
                mn.mi_norm_bwd(probs[s_ % nsets], sh)
            else:
                mn.mi_norm_bwd_variant(vid, probs[s_ % nsets], sh)

    # -- parity gate on set 0
    with torch.cuda.stream(stream):
        run_python(1)
    torch.cuda.synchronize()
    ref = (oracle.layernorm_bwd16(dy_h, x_h, fmt, p0_h, mean_h, rstd_h) if (ln and fmt) else
           oracle.rmsnorm_bwd16(dy_h, x_h, fmt, p0_h, rstd_h) if fmt else
           oracle.layernorm_bwd(dy_h, x_h, p0_h, mean_h, rstd_h) if ln else
           oracle.rmsnorm_bwd(dy_h, x_h, p0_h, rstd_h))
    sample = np.arange(rows) if rows * d <= (1 << 26) else np.unique(np.random.default_rng(0).integers(0, rows, 512))
    got = dxs[0].cpu()
    got = got.view(torch.int16).numpy().view(np.uint16) if es == 2 else got.numpy()
    ok, err, ratio = oracle.dx_tolerance_ok(np.ascontiguousarray(got[sample]), ref["dx64"][sample],
                                            ref["dx_scale"][sample], fmt)
    grads = [(dgs[0], "dgamma" if ln else "dw")] + ([(dbs[0], "dbeta")] if ln else [])
    for t, key in grads:
        o2, e2, r2 = oracle.colsum_tolerance_ok(t.cpu().numpy(), ref[key + "64"], ref["abs_" + key])
        ok, err, ratio = ok and o2, max(err, e2), max(ratio, r2)
    if not ok:
        print(f"PARITY FAILURE before timing: max abs err {err:.3e}, err/bound {ratio:.3f}", file=sys.stderr)
        return 3
    parity = {"rows_checked": int(len(sample)), "max_abs_err": err, "max_err_over_bound": ratio}

    def cpu_fn(budget, threads):
        def call():
            if fmt:
                return (oracle.layernorm_bwd16(dy_h, x_h, fmt, p0_h, mean_h, rstd_h) if ln
                        else oracle.rmsnorm_bwd16(dy_h, x_h, fmt, p0_h, rstd_h))
            return (oracle.layernorm_bwd(dy_h, x_h, p0_h, mean_h, rstd_h) if ln
                    else oracle.rmsnorm_bwd(dy_h, x_h, p0_h, rstd_h))
        return time_oracle(call, budget, threads)

    return measure_and_print(args, torch, stream, run_native, run_python, rotated, nsets, per_set, variant_name,
                             algorithmic_bytes(op_b, rows, d, False, storage), parity,
                             None if args.no_cpu_baseline else cpu_fn,
                             describe(op_b, rows, d, False, storage, pad),
                             {"rows": rows, "d": d, "row_stride": ld, "storage": storage, "eps": eps,
                              "pattern": pattern, "seed": seed, "workspace_bytes": nbytes}, rows)


def bench_calib(args, torch, np, mn, dev, wk) -> int:
    """The parts of a launch (mi_calib_launch): an empty kernel, a read-only
    and a write-only pass over rotated buffers, timed like a step."""
    op, _, rows, d, _, _, _ = wk
    kind = {"empty": 0, "read": 1, "write": 2}[op]
    BL = load_bench_lib()
    n = rows * d
    per_set = 4 * n
    nsets = 1 if (args.mode == "warm" or kind == 0) else max(1, math.ceil(args.footprint_gib * 2**30 / per_set))
    bufs = [torch.zeros(n, device=dev) for _ in range(nsets)] if kind else []
    torch.cuda.synchronize()
    stream = torch.cuda.Stream(device=dev)
    sh = stream.cuda_stream

    def rotated(first: int):
        return (ptr_array(bufs[first:] + bufs[:first]),) if kind else (None,)

    base = rotated(0)

    def run_native(k: int, arrays=None):
        a = (arrays or base)[0]
        st = BL.mi_bench_calib_loop(kind, a if kind == 1 else None, a if kind == 2 else None, nsets, n, k, sh)
        if st != 0:
            raise RuntimeError(f"calibration loop failed: {mn.mi_norm_status_string(st)}")

    def run_python(k: int, start: int = 0):
        for s_ in range(start, start + k):
            b = bufs[s_ % nsets] if kind else None
            mn.mi_calib_launch(kind, b if kind == 1 else None, b if kind == 2 else None, n, stream=sh)

    with torch.cuda.stream(stream):
        run_python(1)
    torch.cuda.synchronize()
    if kind == 2 and not bool((bufs[0] == 1.0).all()):
        print("PARITY FAILURE: the write-only pass left other values", file=sys.stderr)
        return 3
    name = {0: "calib_empty", 1: "read_cover", 2: "write_cover"}[kind]
    return measure_and_print(args, torch, stream, run_native, run_python, rotated, nsets, per_set, name,
                             algorithmic_bytes(op, rows, d, False), {"exact": True}, None,
                             describe(op, rows, d, False), {"rows": rows, "d": d, "storage": "f32"},
                             max(rows, 1))


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="ln_4096x768", choices=sorted(BENCH_WORKLOADS))
    ap.add_argument("--mode", default="rotate", choices=["rotate", "warm"])
    ap.add_argument("--launch", default="native", choices=["native", "graph", "python"])
    ap.add_argument("--variant", default=None, help="force a kernel variant by name")
    ap.add_argument("--footprint-gib", type=float, default=1.0)
    ap.add_argument("--cpu-seconds", type=float, default=2.0,
                    help="wall-clock budget of the CPU baseline (all host threads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy", action="store_true",
                    help="skip the calibration copy of the step's bytes")
    ap.add_argument("--profile", action="store_true",
                    help="the run a kernel tracer or counter pass wraps: the parity call, W warm-up "
                         "steps and one span of K steps, nothing else (no copy, no single launches, "
                         "no CPU baseline)")
    ap.add_argument("--kernarg", default="device", choices=["device", "host"],
                    help="where HIP places kernel arguments (HIP_FORCE_DEV_KERNARG=1 or 0, set before "
                         "the HIP runtime starts)")
    args = ap.parse_args(argv)
    os.environ["HIP_FORCE_DEV_KERNARG"] = "1" if args.kernarg == "device" else "0"

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "rows shard across GPUs with no communication, and this build measures one GPU's share.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import row_wise_normalization_layernorm_amd as mn
    from row_wise_normalization_layernorm_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    wk = BENCH_WORKLOADS[args.workload]
    if wk.op.endswith("_bwd"):
        return bench_bwd(args, torch, np, mn, wl, dev, wk)
    if wk.op in ("empty", "read", "write"):
        return bench_calib(args, torch, np, mn, dev, wk)
    op, storage, rows, d, pattern, stats, pad = wk
    eps = wl.EPS
    add = op.startswith("add_")
    ln = op.endswith("layernorm")
    es = ESIZE[storage]
    ld = d + pad
    dtcode = {"f32": mn.MI_NORM_F32, "f16": mn.MI_NORM_F16, "bf16": mn.MI_NORM_BF16}[storage]
    tdtype = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[storage]
    general = storage != "f32" or pad != 0   # the named float32 calls cover the rest
    BL = load_bench_lib()
    mn.lib()

    # -- inputs, resident in HBM before timing
    seed = wl.case_seed(2, rows, d, pattern)
    x_h = wl.make_x(rows, d, pattern, seed)
    r_h = wl.make_x(rows, d, "normal", [6] + seed) if add else None
    if storage != "f32":
        fmt = wl.F16 if storage == "f16" else wl.BF16
        x_h = wl.quantize16(x_h, fmt)
        r_h = wl.quantize16(r_h, fmt) if add else None
    if op == "copy":
        params_h = ()
    elif ln:
        params_h = wl.make_affine(d, [2, d, 99])
    else:
        params_h = (wl.make_weight(d, [2, d, 99]),)
    n = rows * d
    per_set = (4 if add else 2) * es * rows * ld + (8 * rows if stats else 0)
    nsets = 1 if args.mode == "warm" else max(1, math.ceil(args.footprint_gib * 2**30 / per_set))

    def device_rows(host):
        """[rows, d] on the device inside a [rows, ld] buffer (padding unused)."""
        t = torch.from_numpy(host.view(np.int16) if es == 2 else host).to(dev)
        t = t.view(tdtype) if es == 2 else t
        if pad == 0:
            return t
        buf = torch.zeros(rows, ld, dtype=tdtype, device=dev)
        buf[:, :d].copy_(t)
        return buf[:, :d]

    def empty_rows():
        return torch.empty(rows, ld, dtype=tdtype, device=dev)[:, :d]

    x0 = device_rows(x_h)
    xs = [x0] + [device_rows(x_h) for _ in range(nsets - 1)]
    ys = [empty_rows() for _ in range(nsets)]
    rs_, hs = None, None
    if add:
        rs_ = [device_rows(r_h) for _ in range(nsets)]
        hs = [empty_rows() for _ in range(nsets)]
    means = [torch.empty(rows, device=dev) for _ in range(nsets)] if (stats and ln) else None
    rstds = [torch.empty(rows, device=dev) for _ in range(nsets)] if (stats and op != "copy") else None
    params = [torch.from_numpy(p_).to(dev) for p_ in params_h]
    # every buffer above was filled on torch's current stream; the kernels run on
    # their own stream, so make the set-up complete before anything is launched
    torch.cuda.synchronize()

    opcode = {"layernorm": mn.OP_LAYERNORM, "rmsnorm": mn.OP_RMSNORM,
              "add_layernorm": mn.OP_ADD_LAYERNORM, "add_rmsnorm": mn.OP_ADD_RMSNORM}.get(op)
    vid = -1
    if args.variant:
        names = [mn.mi_norm_variant_name(i) for i in range(mn.mi_norm_variant_count())]
        if args.variant not in names:
            print(f"unknown variant {args.variant}", file=sys.stderr)
            return 1
        vid = names.index(args.variant)

    def problem_for(j: int):
        return mn.problem(opcode, rows, d, xs[j], ys[j], params[0], params[1] if ln else None,
                          r=rs_[j] if add else None, h=hs[j] if add else None, dtype=dtcode,
                          ldx=ld, ldr=ld if add else 0, ldy=ld, ldh=ld if add else 0, eps=eps,
                          mean=means[j] if means else None, rstd=rstds[j] if rstds else None)

    if op != "copy":
        probs = [problem_for(j) for j in range(nsets)]
        sel = vid if vid >= 0 else mn.mi_norm_select(probs[0])
        variant_name = mn.mi_norm_variant_name(sel)
    else:
        variant_name = "copy_cover"

    stream = torch.cuda.Stream(device=dev)
    sh = stream.cuda_stream
    xa, ya = ptr_array(xs), ptr_array(ys)
    ra = ptr_array(rs_) if add else None
    ha = ptr_array(hs) if add else None
    ma = ptr_array(means) if means else None
    sa = ptr_array(rstds) if rstds else None
    p0 = params[0].data_ptr() if params else None
    p1 = params[1].data_ptr() if ln else None

    def rot(ts, first):
        return None if ts is None else ptr_array(ts[first:] + ts[:first])

    def rotated(first: int):
        """The pointer arrays starting at buffer set `first`."""
        return (rot(xs, first), rot(ys, first), rot(rs_, first), rot(hs, first), rot(means, first),
                rot(rstds, first))

    def run_native(k: int, arrays=None):
        nonlocal xa, ya, ra, ha, ma, sa
        if arrays is not None:
            saved = xa, ya, ra, ha, ma, sa
            xa, ya, ra, ha, ma, sa = arrays
            try:
                run_native(k)
            finally:
                xa, ya, ra, ha, ma, sa = saved
            return
        if op == "copy":
            st = BL.mi_bench_copy_loop(xa, ya, nsets, n, k, sh)
        elif general:
            st = BL.mi_bench_norm_loop(ctypes.byref(probs[0]), xa, ra, ya, ha, ma, sa, nsets, k, vid, sh)
        elif op == "layernorm":
            st = BL.mi_bench_layernorm_loop(xa, p0, p1, ya, ma, sa, nsets, rows, d, eps, k, vid, sh)
        elif op == "rmsnorm":
            st = BL.mi_bench_rmsnorm_loop(xa, p0, ya, sa, nsets, rows, d, eps, k, vid, sh)
        elif op == "add_layernorm":
            st = BL.mi_bench_add_layernorm_loop(xa, ra, p0, p1, ya, ha, ma, sa, nsets, rows, d, eps, k,
                                                vid, sh)
        else:
            st = BL.mi_bench_add_rmsnorm_loop(xa, ra, p0, ya, ha, sa, nsets, rows, d, eps, k, vid, sh)
        if st != 0:
            raise RuntimeError(f"bench loop failed: {mn.mi_norm_status_string(st)}")

    def run_python(k: int, start: int = 0):
        for s_ in range(start, start + k):
            j = s_ % nsets
            if op == "copy":
                mn.mi_copy_f32(xs[j], ys[j], n, stream=sh)
            elif vid < 0:
                mn.mi_norm_fwd(probs[j], sh)
            else:
                mn.mi_norm_fwd_variant(vid, probs[j], sh)

    # -- parity gate on set 0 (the first call of the run)
    with torch.cuda.stream(stream):
        run_python(1)
    torch.cuda.synchronize()

    def host_rows(t):
        a_ = t.cpu()
        return a_.view(torch.int16).numpy().view(np.uint16) if es == 2 else a_.numpy()

    if op != "copy":
        import oracle
        sample = np.arange(rows) if n <= (1 << 26) else np.unique(
            np.random.default_rng(0).integers(0, rows, 512))
        xs_h = np.ascontiguousarray(x_h[sample])
        rs_h = np.ascontiguousarray(r_h[sample]) if add else None
        ref_y, ref_h, ref_stats = oracle_call(op, xs_h, rs_h, params_h, eps, storage)
        got_y = host_rows(ys[0])[sample]
        if storage == "f32":
            ok, err, ratio = oracle.tolerance_ok(got_y, ref_y)
        else:
            ok, err, ratio = oracle.tolerance_ok16(np.ascontiguousarray(got_y), ref_y,
                                                   oracle.FMT_F16 if storage == "f16" else oracle.FMT_BF16)
        if stats:
            got_stats = [means[0], rstds[0]] if ln else [rstds[0]]
            for got_t, want in zip(got_stats, ref_stats):
                o2, e2, r2 = oracle.tolerance_ok(got_t.cpu().numpy()[sample], want)
                ok, err, ratio = ok and o2, max(err, e2), max(ratio, r2)
        if add:
            got_h = host_rows(hs[0])[sample]
            same = np.array_equal(got_h.view(np.uint16 if es == 2 else np.uint32),
                                  ref_h.view(np.uint16 if es == 2 else np.uint32))
            ok = ok and same
        if not ok:
            print(f"PARITY FAILURE before timing: max abs err {err:.3e}, err/bound {ratio:.3f}", file=sys.stderr)
            return 3
        parity = {"rows_checked": int(len(sample)), "max_abs_err": err, "max_err_over_bound": ratio}
    else:
        if not torch.equal(ys[0], xs[0]):
            print("PARITY FAILURE: copy mismatch", file=sys.stderr)
            return 3
        parity = {"exact": True}

    cpu_fn = None
    if not args.no_cpu_baseline and op != "copy":
        def cpu_fn(budget, threads):
            return cpu_baseline(op, x_h, r_h, params_h, eps, budget, storage, threads)
    return measure_and_print(args, torch, stream, run_native, run_python, rotated, nsets, per_set, variant_name,
                             algorithmic_bytes(op, rows, d, stats, storage), parity, cpu_fn,
                             describe(op, rows, d, stats, storage, pad),
                             {"rows": rows, "d": d, "row_stride": ld, "storage": storage, "eps": eps,
                              "pattern": pattern, "seed": seed}, rows)


if __name__ == "__main__":
    sys.exit(main())
