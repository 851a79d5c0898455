"""GPU parity at shapes where each of the dispatcher's row-count rules fires.

The variants themselves are covered one by one elsewhere; these cases run
the library's own choice (mi_norm_fwd, no forced variant) at the geometry
that makes each rule pick it, with ragged last workgroups, and check the
outputs against the float64 oracle with the bounds of test_parity_storage.
The expected variant names pin the host rules: a change in what the
dispatcher picks shows here before any timing does.
"""
from __future__ import annotations

import pytest

import row_wise_normalization_layernorm_amd as mn
from test_parity_storage import inputs, run_case, say, torch_dev  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

F32, F16, BF16 = mn.MI_NORM_F32, mn.MI_NORM_F16, mn.MI_NORM_BF16
OPS = {"layernorm": mn.OP_LAYERNORM, "rmsnorm": mn.OP_RMSNORM,
       "add_layernorm": mn.OP_ADD_LAYERNORM, "add_rmsnorm": mn.OP_ADD_RMSNORM}

CASES = [
    # workgroups spread evenly over the CUs: 4-wave workgroups where 16-wave
    # ones would load half the CUs twice
    ("layernorm", F32, 6144, 768, "ln_4_p0_l64_w1_q3_b4"),
    ("rmsnorm", F32, 5001, 768, "rms_4_p0_l64_w1_q3_b4"),
    # float32 LayerNorm rows of 3-4 K elements, 3072-4096 rows: sixteen slots
    ("layernorm", F32, 3072, 4096, "ln_4_p0_l64_w1_q16_b4"),
    ("layernorm", F32, 3501, 3584, "ln_4_p0_l64_w1_q16_b8"),
    # float32 one-row rows of 2-4 K elements with many rows: half the waves
    ("rmsnorm", F32, 2561, 4096, "rms_4_p0_l64_w2_q8_b4"),
    ("layernorm", F32, 4097, 3072, "ln_4_p0_l64_w2_q6_b4"),
    ("layernorm", F32, 6145, 2048, "ln_4_p0_l64_w1_q8_b4"),
    # 16-bit rows of two waves with 2560-8192 rows: one wave, twice the slots
    ("layernorm", BF16, 2561, 4096, "ln_bf16_8_p0_l64_w1_q8_b16"),
    ("add_layernorm", F16, 4095, 3072, "addln_f16_8_p0_l64_w1_q6_b16"),
    ("rmsnorm", BF16, 3584, 3584, "rms_bf16_8_p0_l64_w1_q8_b16"),
    ("layernorm", BF16, 5001, 3000, "ln_bf16_8_p0_l64_w1_q6_b4"),      # 16-wave grid uneven
    ("add_rmsnorm", F16, 5003, 4096, "addrms_f16_8_p0_l64_w4_q2_b16"),  # fused, four slots: four waves
    # 16-bit rows of two waves and three or four slots under 2560 rows: multi-row
    ("rmsnorm", BF16, 2049, 4096, "rms_bf16_8_r2_w2_q4_b4"),
    ("add_layernorm", F16, 2049, 3072, "addln_f16_8_r2_w2_q3_b4"),
    # 16-bit rows of four waves from 2048 rows, one-row path: two waves, twice the slots
    ("layernorm", BF16, 2049, 4608, "ln_bf16_8_p0_l64_w2_q6_b16"),
    ("add_rmsnorm", F16, 2051, 8192, "addrms_f16_8_p0_l64_w2_q8_b16"),
    # 16-bit rows of one wave: 4-wave workgroups
    ("add_rmsnorm", BF16, 6145, 2048, "addrms_bf16_8_p0_l64_w1_q4_b4"),
    # fused float32 rows of four waves, 2048-4095 rows: multi-row, two waves, twice the slots
    ("add_layernorm", F32, 3001, 3000, "addln_4_r2_w2_q6_b4"),
    # float32 RMSNorm rows of two waves, 2048-4096 rows: the base shape
    ("rmsnorm", F32, 3001, 1800, "rms_4_p0_l64_w2_q4_b4"),
    # fused float32 rows of two waves up to 4096 rows: one wave of eight slots
    ("add_layernorm", F32, 2049, 1536, "addln_4_p0_l64_w1_q8_b4"),
    ("add_rmsnorm", F32, 4095, 2048, "addrms_4_p0_l64_w1_q8_b4"),
    # peeled rows of fewer than eight waves: the fewest waves that hold them in
    # four slots, the largest workgroups that still give every CU one
    ("layernorm", F32, 1023, 2049, "ln_4_p1_l64_w2_q4_b4"),
    ("rmsnorm", F32, 1021, 4097, "rms_4_p1_l64_w4_q4_b16"),
    ("layernorm", BF16, 1001, 4100, "ln_bf16_8_p1_l64_w2_q4_b4"),
    # many rows: two rows per wave group, the base shape's waves and slots
    ("layernorm", F32, 8193, 4096, "ln_4_r2_w4_q4_b4"),
    ("rmsnorm", F32, 8193, 3072, "rms_4_r2_w4_q3_b4"),
    # fused rows of four or eight waves with many rows: twice the waves
    ("add_layernorm", F32, 8193, 4096, "addln_4_p0_l64_w8_q2_b16"),
    ("add_rmsnorm", BF16, 8193, 8192, "addrms_bf16_8_p0_l64_w8_q2_b16"),
]


def _chosen(op, dt, rows, d):
    base = 1 << 40
    ln, add = op.endswith("layernorm"), op.startswith("add_")
    p = mn.problem(OPS[op], rows, d, base, base + (1 << 36), base + (2 << 36),
                   base + (2 << 36) + (1 << 20) if ln else None,
                   r=base + (3 << 36) if add else None, h=base + (4 << 36) if add else None, dtype=dt)
    return mn.mi_norm_variant_name(mn.mi_norm_select(p))


@pytest.mark.parametrize("op,dt,rows,d,name", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}x{c[3]}" for c in CASES])
def test_dispatch_rule_shapes(torch_dev, op, dt, rows, d, name):
    torch, dev = torch_dev
    assert _chosen(op, dt, rows, d) == name
    say(f"dispatch rule {op} dt={dt} [{rows}x{d}] -> {name}")
    x, r, params = inputs(op, dt, rows, d, "offset", [31, rows, d])
    run_case(torch, dev, op, dt, x, r, params)
