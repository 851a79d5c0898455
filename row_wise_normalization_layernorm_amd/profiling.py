"""Summarize rocprofv3 output (kernel trace + stats, or counter collection).

    python -m row_wise_normalization_layernorm_amd.profiling trace DIR PREFIX [--skip S] [--last N]
    python -m row_wise_normalization_layernorm_amd.profiling pmc DIR PREFIX COUNTER

``trace`` reads ``PREFIX_kernel_stats.csv`` and ``PREFIX_kernel_trace.csv``
(``rocprofv3 --kernel-trace --stats --output-format csv``) and prints, per
kernel, the dispatch count and the mean/median/min/max duration over N
dispatches after the first S (a bench run's timed steps: S = 1 parity call +
the warm-up steps, N = the timed steps).  ``pmc`` reads
``PREFIX_counter_collection.csv`` and prints the per-dispatch mean of a
counter, per kernel.
"""
from __future__ import annotations

import argparse
import csv
import os
import statistics
import sys
from collections import defaultdict


def _short(name: str) -> str:
    return name.replace("minorm::", "").replace("(minorm::NormParams)", "")


def trace_summary(directory: str, prefix: str, last: int, skip: int = 0) -> str:
    rows = list(csv.DictReader(open(os.path.join(directory, f"{prefix}_kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    per = defaultdict(list)
    for r in rows:
        per[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = ["kernel | dispatches | window | mean us | median us | min us | max us"]
    for name, ds in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        tail = ds[skip:skip + last] if last else ds[skip:]
        tail = tail or ds
        out.append(f"{_short(name)} | {len(ds)} | {len(tail)} | {statistics.mean(tail) / 1e3:.3f} | "
                   f"{statistics.median(tail) / 1e3:.3f} | {min(tail) / 1e3:.3f} | {max(tail) / 1e3:.3f}")
    stats = os.path.join(directory, f"{prefix}_kernel_stats.csv")
    if os.path.exists(stats):
        out.append("")
        out.append("rocprofv3 --stats (all dispatches):")
        for r in csv.DictReader(open(stats)):
            out.append(f"  {_short(r['Name'])}: calls {r['Calls']}, average {float(r['AverageNs']) / 1e3:.3f} us, "
                       f"min {float(r['MinNs']) / 1e3:.3f} us, max {float(r['MaxNs']) / 1e3:.3f} us")
    return "\n".join(out)


def pmc_means(directory: str, prefix: str, counter: str) -> dict:
    rows = list(csv.DictReader(open(os.path.join(directory, f"{prefix}_counter_collection.csv"))))
    per = defaultdict(list)
    for r in rows:
        if r.get("Counter_Name") == counter:
            per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: (statistics.mean(v), len(v)) for k, v in per.items()}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("prefix")
    t.add_argument("--last", type=int, default=0, help="dispatches in the window (0: all after --skip)")
    t.add_argument("--skip", type=int, default=0, help="dispatches before the window")
    p = sub.add_parser("pmc")
    p.add_argument("dir")
    p.add_argument("prefix")
    p.add_argument("counter")
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        print(trace_summary(a.dir, a.prefix, a.last, a.skip))
    else:
        for k, (m, n) in pmc_means(a.dir, a.prefix, a.counter).items():
            print(f"{_short(k)} | {a.counter} mean {m:.1f} over {n} dispatches")
    return 0


if __name__ == "__main__":
    sys.exit(main())
