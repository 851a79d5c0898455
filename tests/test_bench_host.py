"""bench.py's host logic on the CPU: the algorithmic byte counts, the pairing
of committed counter summaries with the current kernels, and the one-GPU
rule.  Nothing here touches a device."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes():
    ab = bench.algorithmic_bytes
    # forward: read x + write y, gamma/beta, mean/rstd
    assert ab("layernorm", 4096, 768, True) == 8 * 4096 * 768 + 8 * 768 + 8 * 4096 == 25204736
    assert ab("layernorm", 32768, 8192, False) == 8 * 32768 * 8192 + 8 * 8192
    assert ab("rmsnorm", 2048, 4096, False) == 8 * 2048 * 4096 + 4 * 4096
    assert ab("rmsnorm", 256, 8193, True) == 8 * 256 * 8193 + 4 * 8193 + 4 * 256
    # fused: x, r read and y, h written
    assert ab("add_layernorm", 4096, 768, True) == 16 * 4096 * 768 + 8 * 768 + 8 * 4096
    # 16-bit rows halve the row terms only
    assert ab("layernorm", 32768, 8192, False, "bf16") == 4 * 32768 * 8192 + 8 * 8192
    assert ab("add_rmsnorm", 4096, 768, False, "f16") == 8 * 4096 * 768 + 4 * 768
    # backward: dy, x read, dx written; gamma read, dgamma/dbeta written; mean/rstd read
    assert ab("layernorm_bwd", 4096, 768, False) == 12 * 4096 * 768 + 12 * 768 + 8 * 4096
    assert ab("rmsnorm_bwd", 8192, 8192, False) == 12 * 8192 * 8192 + 8 * 8192 + 4 * 8192
    assert ab("layernorm_bwd", 32768, 8192, False, "bf16") == 6 * 32768 * 8192 + 12 * 8192 + 8 * 32768
    assert ab("copy", 4096, 768, False) == 8 * 4096 * 768


def test_every_workload_is_described_and_sized():
    for name, wk in bench.BENCH_WORKLOADS.items():
        if wk.op == "empty":
            assert bench.algorithmic_bytes(wk.op, wk.rows, wk.d, wk.stats) == 0
            assert "empty kernel" in bench.describe(wk.op, wk.rows, wk.d, wk.stats)
            continue
        assert bench.algorithmic_bytes(wk.op, wk.rows, wk.d, wk.stats, wk.storage) > 0, name
        desc = bench.describe(wk.op, wk.rows, wk.d, wk.stats, wk.storage, wk.pad)
        assert f"[{wk.rows},{wk.d}]" in desc or "bytes of" in desc, (name, desc)
        assert bench.direction_of(name) == ("bwd" if wk.op.endswith("_bwd") else "fwd")
    # the default workload is the headline: LayerNorm FP32 [4096,768] with mean/rstd
    assert bench.BENCH_WORKLOADS["ln_4096x768"] == bench.W("layernorm", "f32", 4096, 768, "normal", True)


def test_trace_pairing(tmp_path, monkeypatch):
    """Per-dispatch kernel times count only for the kernel sources and the
    variant the trace was taken with, as the counters do."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    for rel in set(bench.KERNEL_SOURCES["fwd"] + bench.KERNEL_SOURCES["bwd"]):
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, rel), "rb").read())
    h = bench.kernel_source_hash("fwd")
    f = tmp_path / "profiles" / "ln_4096x768.txt"
    body = ("dispatch_us_median: 5.3\ndispatch_us_min: 4.9\ndispatch_us_max: 6.7\n"
            "dispatch_us_mean: 5.6\ndispatches: 100\n")
    f.write_text(f"kernel_variant: ln_4_p0_l64_w1_q3_b16\nkernel_source_sha256: {h}\n" + body)
    got = bench.trace_stats("ln_4096x768", "ln_4_p0_l64_w1_q3_b16")
    assert got["median"] == 5.3 and got["min"] == 4.9 and got["max"] == 6.7 and got["dispatches"] == 100
    assert bench.trace_stats("ln_4096x768", "ln_4_p0_l64_w1_q3_b4") is None        # another variant
    f.write_text("kernel_variant: ln_4_p0_l64_w1_q3_b16\nkernel_source_sha256: 0000000000000000\n" + body)
    assert bench.trace_stats("ln_4096x768", "ln_4_p0_l64_w1_q3_b16") is None       # kernels changed
    assert bench.trace_stats("rms_4096x768", "x") is None                           # no trace


def test_profile_pairing(tmp_path, monkeypatch):
    """A counter summary counts only for the kernel sources and the variant it was taken with."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    # the hash is computed from the sources under ROOT: copy them
    for rel in set(bench.KERNEL_SOURCES["fwd"] + bench.KERNEL_SOURCES["bwd"]):
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, rel), "rb").read())
    h = bench.kernel_source_hash("fwd")
    f = tmp_path / "profiles" / "ln_4096x768.txt"
    f.write_text(f"kernel_variant: ln_4_p0_l64_w1_q3_b16\nkernel_source_sha256: {h}\n"
                 "traffic_bytes_per_launch: 25264977\n")
    assert bench.pmc_traffic("ln_4096x768", "ln_4_p0_l64_w1_q3_b16")[0] == 25264977
    assert bench.pmc_traffic("ln_4096x768", "ln_4_p0_l64_w1_q3_b4")[0] is None      # another variant
    f.write_text("kernel_variant: ln_4_p0_l64_w1_q3_b16\nkernel_source_sha256: 0000000000000000\n"
                 "traffic_bytes_per_launch: 25264977\n")
    assert bench.pmc_traffic("ln_4096x768", "ln_4_p0_l64_w1_q3_b16")[0] is None      # kernels changed
    assert bench.pmc_traffic("ln_512x128", "x")[0] is None                            # no summary
    # the backward's hash follows the backward's sources, not the forward's
    assert bench.kernel_source_hash("bwd") != h


def test_code_text_drops_comments_only():
    src = ('// head\nint a = 1; /* two\nlines */ const char *s = "x // y /* z */";\n'
           "char c = '/'; int b = a / 2;  // tail\n")
    assert bench.code_text(src) == ("int a = 1; const char *s = \"x // y /* z */\"; "
                                    "char c = '/'; int b = a / 2;")
    # a change of code is seen, a change of comment or spacing is not
    assert bench.code_text("x = a + b; // sum") == bench.code_text("x = a +  b;\n// the sum")
    assert bench.code_text("x = a + b;") != bench.code_text("x = a - b;")


def test_committed_profiles_name_their_command_and_kernel():
    prof = os.path.join(ROOT, "profiles")
    for name in os.listdir(prof):
        text = open(os.path.join(prof, name)).read()
        assert "rocprofv3" in text and "bench.py" in text, name
        if name.startswith("pmc_"):
            assert "kernel_variant:" in text and "traffic_bytes_per_launch:" in text, name
            workload = name[len("pmc_"):-len(".txt")]
            assert workload in bench.BENCH_WORKLOADS, name


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


class _FakeTorch:
    """Just enough of torch.cuda for gated_span: the start event reads as
    already completed (the gate ran out) for the first ``late`` runs."""

    def __init__(self, late):
        self.late, self.sleeps, self.records = late, [], 0
        fake = self

        class Event:
            def __init__(self, enable_timing=False):
                self.n = None

            def record(self, stream):
                fake.records += 1
                self.n = fake.records

            def query(self):
                return len(fake.sleeps) <= fake.late

            def elapsed_time(self, other):
                return float(other.n - self.n)

        class _Ctx:
            def __enter__(self):
                return self

            def __exit__(self, *a):
                return False

        class cuda:
            pass

        cuda.Event = Event
        cuda.synchronize = staticmethod(lambda: None)
        cuda.stream = staticmethod(lambda s: _Ctx())
        cuda._sleep = staticmethod(lambda c: fake.sleeps.append(c))
        self.cuda = cuda


def test_gate_repeats_the_span_until_it_covers_the_launches():
    queued = []
    t = _FakeTorch(late=2)
    ms, wall, gate_us, covered = bench.gated_span(t, None, 100, lambda: queued.append(1))
    g = bench.gate_cycles(100)
    assert t.sleeps == [g, 2 * g, 4 * g] and len(queued) == 3 and covered
    assert gate_us == 4 * g / 2400 and ms == 1.0
    t = _FakeTorch(late=9)
    _, _, gate_us, covered = bench.gated_span(t, None, 100, lambda: None, tries=4)
    assert len(t.sleeps) == 4 and not covered and gate_us == 8 * g / 2400
    t = _FakeTorch(late=0)
    bench.gated_span(t, None, 100, lambda: None)
    assert t.sleeps == [g]
