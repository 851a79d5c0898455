"""Compile the C reference oracle (ref_norm.c) into liboracle_norm.so with gcc.

Test infrastructure: the oracle is the checker, never the product path.
``plant`` builds a copy with one deliberate mistake for the negative-control
tests (see ORACLE_PLANT in ref_norm.c); those copies go to a caller-chosen
directory and are never loaded by anything but those tests.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ref_norm.c")
LIB = os.path.join(HERE, "liboracle_norm.so")


def build(out: str = LIB, plant: int = 0, verbose: bool = False) -> str:
    """Build the oracle shared library and return its path."""
    cmd = [
        "gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
        # strict IEEE double evaluation: no fast-math, no FMA contraction,
        # so each float64 operation rounds exactly once as written
        "-ffp-contract=off", "-fno-fast-math",
        f"-DORACLE_PLANT={int(plant)}",
        SRC, "-o", out + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
