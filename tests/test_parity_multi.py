"""GPU tests of the multi-row variants (two rows per wave group sharing one
fetch of the parameters): the same bits as the one-row variant of the same
shape, in place and with h written over an input, and the dispatcher's
choice of them for many rows.  Every compiled multi-row variant is also
checked against the oracle by test_parity.test_every_variant (float32) and
test_parity_storage.test_every_variant_strided (every storage type)."""
from __future__ import annotations

import numpy as np
import pytest

import row_wise_normalization_layernorm_amd as mn
from row_wise_normalization_layernorm_amd import workloads as wl
from test_parity_storage import DT16, FMT, OPNAME, inputs, run_case, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    mn.lib()
    return torch, torch.device("cuda:0")


def _infos():
    return [(i, mn.mi_norm_variant_name(i), mn.mi_norm_variant_get_info(i))
            for i in range(mn.mi_norm_variant_count())]


def _one_row_twin(infos, v):
    """A one-row held variant with the multi-row variant's operation, storage
    type and (waves per row, slots)."""
    for i, _, u in infos:
        if (u["op"], u["dtype"], u["vec"], u["waves_per_row"], u["slots"]) == \
                (v["op"], v["dtype"], v["vec"], v["waves_per_row"], v["slots"]) and \
                u["rows_per_lane"] == 1 and not u["peel"] and not u["looped"] and u["lanes_per_row"] == 64:
            return i
    return None


def _bits(t):
    import torch
    a = t.cpu()
    return a.view(torch.int32 if a.element_size() == 4 else torch.int16).numpy()


def test_multi_row_matches_one_row_bit_for_bit(torch_dev):
    """The kernels sum, merge and normalize in the same order, so outputs,
    statistics and h agree in every bit, also on a ragged last row group and
    a ragged last slot."""
    torch, dev = torch_dev
    infos = _infos()
    multi = [(i, n, v) for i, n, v in infos if v["rows_per_lane"] == 2]
    # per operation: float32 one wave 1-4 slots, two waves 3, 4, 6, 8, four and
    # eight waves 3, 4 (12); each 16-bit type two, four, eight waves 3, 4 (6)
    assert len(multi) == 4 * (12 + 2 * 6)
    tdt = {mn.MI_NORM_F32: torch.float32, mn.MI_NORM_F16: torch.float16, mn.MI_NORM_BF16: torch.bfloat16}
    stream = torch.cuda.current_stream().cuda_stream
    for vid, name, v in multi:
        twin = _one_row_twin(infos, v)
        assert twin is not None, name
        op, dt = OPNAME[v["op"]], v["dtype"]
        ln, add = op.endswith("layernorm"), op.startswith("add_")
        cap, step = v["max_d"], v["vec"]
        for d in sorted({cap, max(step, cap - step * max(1, cap // (7 * step)))}):
            rows = 2 * v["rows_per_block"] + 1
            say(f"bitwise {name} vs {mn.mi_norm_variant_name(twin)} rows={rows} d={d}")
            x, r, params = inputs(op, dt, rows, d, "offset", [21, vid, d])

            def dev_rows(a):
                if a is None:
                    return None
                if dt == mn.MI_NORM_F32:
                    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(tdt[dt])

            X, R = dev_rows(x), dev_rows(r)
            P = [torch.from_numpy(p).to(dev) for p in params]
            outs = []
            for k in (vid, twin):
                Y = torch.empty(rows, d, dtype=tdt[dt], device=dev)
                H = torch.empty(rows, d, dtype=tdt[dt], device=dev) if add else None
                M = torch.empty(rows, device=dev) if ln else None
                S = torch.empty(rows, device=dev)
                prob = mn.problem(v["op"], rows, d, X, Y, P[0], P[1] if ln else None, r=R, h=H, dtype=dt,
                                  eps=wl.EPS, mean=M, rstd=S)
                mn.mi_norm_fwd_variant(k, prob, stream)
                torch.cuda.synchronize()
                outs.append([_bits(t) for t in (Y, H, M, S) if t is not None])
            for a, b in zip(*outs):
                assert np.array_equal(a, b), name


def test_workgroup_twins_match_bit_for_bit(torch_dev):
    """Variants that differ only in their workgroup's size (how many rows a
    workgroup holds) sum, merge and normalize each row in the same order, so
    their outputs agree in every bit.  Among them are the 16-bit rows whose
    larger workgroups stage the parameters in LDS while the one-row
    workgroups fetch them in the output pass: the comparison is the
    regression check on that staging (a 16-byte store followed by an LDS read
    that reuses its data registers)."""
    torch, dev = torch_dev
    infos = _infos()
    groups = {}
    for i, n, v in infos:
        if v["looped"] or v["rows_per_lane"] != 1 or v["op"] not in OPNAME:
            continue                     # backward variants: test_parity_bwd.py
        key = (v["op"], v["dtype"], v["vec"], v["peel"], v["lanes_per_row"], v["waves_per_row"], v["slots"])
        groups.setdefault(key, []).append((i, n, v))
    twins = [g for g in groups.values() if len(g) > 1]
    assert len(twins) > 100
    tdt = {mn.MI_NORM_F32: torch.float32, mn.MI_NORM_F16: torch.float16, mn.MI_NORM_BF16: torch.bfloat16}
    stream = torch.cuda.current_stream().cuda_stream
    checked = 0
    for g in twins:
        _, name0, v = g[0]
        op, dt = OPNAME[v["op"]], v["dtype"]
        ln, add = op.endswith("layernorm"), op.startswith("add_")
        cap, step = min(u["max_d"] for _, _, u in g), v["vec"]
        d = max(step, cap - step * max(1, cap // (7 * step)))
        rows = 2 * max(u["rows_per_block"] for _, _, u in g) + 1
        x, r, params = inputs(op, dt, rows, d, "offset", [23, v["op"], dt, d])

        def dev_rows(a):
            if a is None:
                return None
            if dt == mn.MI_NORM_F32:
                return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(tdt[dt])

        X, R = dev_rows(x), dev_rows(r)
        P = [torch.from_numpy(p).to(dev) for p in params]
        outs = []
        for k, name, _ in g:
            Y = torch.empty(rows, d, dtype=tdt[dt], device=dev)
            H = torch.empty(rows, d, dtype=tdt[dt], device=dev) if add else None
            M = torch.empty(rows, device=dev) if ln else None
            S = torch.empty(rows, device=dev)
            prob = mn.problem(v["op"], rows, d, X, Y, P[0], P[1] if ln else None, r=R, h=H, dtype=dt,
                              eps=wl.EPS, mean=M, rstd=S)
            if not mn.mi_norm_eligible(k, prob):
                continue
            say(f"workgroup twins {name} rows={rows} d={d}")
            mn.mi_norm_fwd_variant(k, prob, stream)
            torch.cuda.synchronize()
            outs.append((name, [_bits(t) for t in (Y, H, M, S) if t is not None]))
        for name, o in outs[1:]:
            for a, b in zip(outs[0][1], o):
                assert np.array_equal(a, b), f"{name} differs from {outs[0][0]}"
            checked += 1
    assert checked > 100


@pytest.mark.parametrize("dt", [pytest.param(mn.MI_NORM_F32, id="f32")] + DT16)
@pytest.mark.parametrize("op", list(OPNAME.values()))
def test_multi_row_in_place_and_aliased(torch_dev, dt, op):
    """An odd row count (a half-filled last row group) at widths of one and
    of several waves per row (16-bit rows: only from four waves per row,
    where the dispatcher picks the multi-row variants), written over the
    input: y over x, and for the fused operations h over x or over r;
    strided rows with gaps."""
    torch, dev = torch_dev
    one_row = op.startswith("add_") or op == "rmsnorm"
    # float32 fused and RMSNorm rows of four waves from 8192 rows run one row
    # per wave group; 4097 rows of 4096 (64 MiB) are multi-row
    shapes = ((8193, 768), (4097 if one_row else 8193, 4096)) if dt == mn.MI_NORM_F32 else ((4097, 8192),)
    for rows, d in shapes:
        x, r, params = inputs(op, dt, rows, d, "offset", [22, d])
        ld = {k: d + 16 for k in "xryh"}
        probe = mn.problem({v: k for k, v in OPNAME.items()}[op], rows, d, 1 << 40, 1 << 41, 1 << 42,
                           (1 << 42) + 65536 if op.endswith("layernorm") else None,
                           r=(1 << 43) if op.startswith("add_") else None,
                           h=(1 << 44) if op.startswith("add_") else None, dtype=dt,
                           ldx=ld["x"], ldr=ld["r"] if op.startswith("add_") else 0, ldy=ld["y"],
                           ldh=ld["h"] if op.startswith("add_") else 0)
        chosen = mn.mi_norm_variant_name(mn.mi_norm_select(probe))
        assert "_r2_" in chosen, chosen
        modes = [dict(y_mode="x")]
        if op.startswith("add_"):
            modes += [dict(h_mode="x"), dict(h_mode="r"), dict(y_mode="r", h_mode="x")]
        for m in modes:
            say(f"multi-row aliased {op} dt={dt} [{rows}x{d}] {chosen} {m}")
            run_case(torch, dev, op, dt, x, r, params, ld=ld, **m)
