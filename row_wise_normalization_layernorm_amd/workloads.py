"""Seeded synthetic inputs for row-wise normalization.

This module only draws and shapes input data; it contains none of the
normalization arithmetic.  Both the GPU path's tests/benchmark and the CPU
oracle are fed from here, so the two sides always see the same float32 bits.

Input patterns follow the correctness protocol of "RMSNorm on an RTX 5070"
(section "Correctness before timing"): normal random values, zeros, small
values and alternating signs.  Readings taken where that page is silent:

* "small" is N(0,1) * 1e-6, scaled in float64 and rounded once to float32;
* "alternating" is +1 at even and -1 at odd positions of the row-major flat
  index, so an odd width starts successive rows on opposite signs;
* "offset" (N(0,1) * 3 + 0.5, float64 then rounded) moves the row mean away
  from zero so that a variance formed as E[x^2] - mu^2 loses digits.

Scale/shift vectors: gamma = 1 + 0.1 N, beta = 0.1 N, RMSNorm weight
w = 1 + 0.1 N, each formed in float64 and rounded once.

Every draw comes from ``numpy.random.default_rng`` (PCG64) seeded with a short
integer list, recorded by the callers next to their results.

16-bit inputs (binary16, bfloat16) are the float32 draws cast by numpy
(binary16) or torch (bfloat16), both round-to-nearest-even library casts,
and are handled as uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PATTERNS = ("normal", "zero", "tiny", "alternating", "offset")
_PATTERN_ID = {p: i for i, p in enumerate(PATTERNS)}

EPS = 1e-5  # the epsilon fixed by "RMSNorm on an RTX 5070", section "The operator and the change"


def case_seed(tag: int, rows: int, d: int, pattern: str) -> list[int]:
    """The seed list for one case: a caller tag, the shape and the pattern."""
    return [int(tag), int(rows), int(d), _PATTERN_ID[pattern]]


def make_x(rows: int, d: int, pattern: str = "normal", seed=0) -> np.ndarray:
    """A C-contiguous float32 [rows, d] input drawn for ``pattern``."""
    if pattern not in _PATTERN_ID:
        raise ValueError(f"unknown pattern {pattern!r}; choose from {PATTERNS}")
    rng = np.random.default_rng(seed)
    if pattern == "zero":
        return np.zeros((rows, d), np.float32)
    if pattern == "alternating":
        flat = np.ones(rows * d, np.float32)
        flat[1::2] = -1.0
        return flat.reshape(rows, d)
    x = rng.standard_normal((rows, d), dtype=np.float32)
    if pattern == "tiny":
        x = (x.astype(np.float64) * 1e-6).astype(np.float32)
    elif pattern == "offset":
        x = (x.astype(np.float64) * 3.0 + 0.5).astype(np.float32)
    return np.ascontiguousarray(x)


F16 = 1   # IEEE binary16 storage
BF16 = 2  # bfloat16 storage
FORMATS = {"f16": F16, "bf16": BF16}


def quantize16(x: np.ndarray, fmt: int) -> np.ndarray:
    """uint16 patterns of float32 ``x`` cast to a 16-bit format by a library cast."""
    x = np.ascontiguousarray(x, np.float32)
    if fmt == F16:
        return x.astype(np.float16).view(np.uint16)
    if fmt == BF16:
        import torch
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(f"unknown 16-bit format {fmt}")


def make_x16(rows: int, d: int, pattern: str, seed, fmt: int) -> np.ndarray:
    """make_x's draw in a 16-bit storage format (uint16 patterns)."""
    return quantize16(make_x(rows, d, pattern, seed), fmt)


def make_affine(d: int, seed=0) -> tuple[np.ndarray, np.ndarray]:
    """LayerNorm scale and shift: gamma ~ N(1, 0.1), beta ~ N(0, 0.1)."""
    rng = np.random.default_rng(seed)
    gamma = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    beta = (0.1 * rng.standard_normal(d)).astype(np.float32)
    return gamma, beta


def make_weight(d: int, seed=0) -> np.ndarray:
    """RMSNorm weight: w ~ N(1, 0.1)."""
    rng = np.random.default_rng(seed)
    return (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)


@dataclass(frozen=True)
class Case:
    op: str            # "layernorm", "rmsnorm", "add_layernorm" or "add_rmsnorm"
    rows: int
    d: int
    pattern: str = "normal"
    stats: bool = False  # also produce per-row mean/rstd (rstd only for RMSNorm)
    tag: int = 0

    @property
    def name(self) -> str:
        return f"{self.op}[{self.rows}x{self.d}]/{self.pattern}"

    def inputs(self):
        """(x, params...) for this case: (x, gamma, beta) or (x, w)."""
        a = self.arrays()
        return (a["x"],) + a["params"]

    def arrays(self) -> dict:
        """x, the residual r (fused ops; None otherwise) and the parameters."""
        seed = case_seed(self.tag, self.rows, self.d, self.pattern)
        x = make_x(self.rows, self.d, self.pattern, seed)
        r = make_x(self.rows, self.d, "normal", [6] + seed) if self.op.startswith("add_") else None
        pseed = [int(self.tag), int(self.d), 99]
        if self.op.endswith("layernorm"):
            params = make_affine(self.d, pseed)
        else:
            params = (make_weight(self.d, pseed),)
        return {"x": x, "r": r, "params": params}


@dataclass(frozen=True)
class Workload:
    name: str
    cases: tuple = field(default_factory=tuple)


_BASIC = ("normal", "zero", "tiny", "alternating")

# The five workload families exercised by tests and benchmark.
WORKLOADS = {
    # LayerNorm [512,128] plus ragged widths 1/31/33/127 at 64 rows, four patterns each
    "ln_small": Workload("ln_small", tuple(
        [Case("layernorm", 512, 128, p, tag=1) for p in _BASIC]
        + [Case("layernorm", 64, d, p, tag=1) for d in (1, 31, 33, 127) for p in _BASIC])),
    # LayerNorm [4096,768] with per-row mean/rstd: the headline shape
    "ln_4096x768": Workload("ln_4096x768", (Case("layernorm", 4096, 768, "normal", True, tag=2),)),
    # LayerNorm shape sweep with an offset mean
    "ln_sweep": Workload("ln_sweep", tuple(
        Case("layernorm", r, d, "offset", tag=3) for r, d in ((8192, 768), (1024, 2048), (4096, 4096)))),
    # RMSNorm shapes x four patterns
    "rms": Workload("rms", tuple(
        Case("rmsnorm", r, d, p, tag=4)
        for r, d in ((512, 128), (4096, 768), (2048, 4096), (256, 8193)) for p in _BASIC)),
    # residual add fused before either norm (the sum h = x + r written out)
    "residual": Workload("residual", tuple(
        [Case("add_layernorm", 4096, 768, "normal", True, tag=6)]
        + [Case("add_layernorm", 64, d, p, True, tag=6) for d in (1, 33, 127, 2049, 8193)
           for p in ("normal", "offset")]
        + [Case("add_rmsnorm", r, d, p, True, tag=6)
           for r, d in ((512, 128), (2048, 4096), (256, 8193)) for p in ("normal", "tiny")])),
    # LayerNorm at bandwidth-saturating scale: 1 GiB read + 1 GiB written
    "ln_32768x8192": Workload("ln_32768x8192", (Case("layernorm", 32768, 8192, "normal", tag=5),)),
}
