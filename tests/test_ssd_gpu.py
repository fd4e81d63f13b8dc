"""Mamba-2 SSD layer on the GPU (ssm_ssd_fwd through the C ABI, chunked
matrix form on bf16 MFMA) against the fp64 oracle's recurrence.

Tolerance: 2e-2 floored max relative error (bf16 inputs, workloads.rel_err).
Besides the inputs' own rounding, the kernel rounds three MFMA operands to
bf16 (the decayed mask M, the weighted x of the state update and the state
copy read by the inter-chunk term), each a relative 2^-9 per element inside
fp32 sums; y is rounded once to bf16.  The fp32 final state is held to the
same bound.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mamba_selective_scan_06_amd as ssm
import oracle
import workloads
from tests.gpu_helpers import DEV, check

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP GPU"),
]

SW = workloads.SSD_WORKLOADS
TENS = ("x", "dt", "A", "B", "C", "D", "dt_bias", "h0")
TOL = workloads.tolerance(torch.bfloat16)


def gpu_ssd(inp):
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    y, hT = ssm.ssd_fwd(*(d[k] for k in TENS), return_final_state=True)
    torch.cuda.synchronize()
    return y.float().cpu().double().numpy(), hT.cpu().double().numpy()


def oracle_ssd(inp):
    return oracle.ssd(*(inp[k] for k in ("x", "dt", "A", "B", "C")), D=inp["D"], dt_bias=inp["dt_bias"],
                      s0=inp["h0"])


CASES = [
    dict(dstate=64, ngroups=2, seqlen=200),
    dict(dstate=128, ngroups=1, seqlen=200),
    dict(dstate=256, ngroups=4, seqlen=130),
    dict(dstate=128, ngroups=2, seqlen=64),   # exactly one chunk
    dict(dstate=128, ngroups=2, seqlen=65),   # one token into the second chunk
    dict(dstate=64, ngroups=1, seqlen=1),
    dict(dstate=64, ngroups=4, seqlen=63),
]


@pytest.mark.parametrize("case", CASES, ids=[f"N{c['dstate']}-G{c['ngroups']}-L{c['seqlen']}" for c in CASES])
@pytest.mark.parametrize("with_h0", [False, True], ids=["zero-state", "h0"])
def test_ssd_small_all_elements(case, with_h0):
    inp = workloads.make_ssd_inputs(SW[0], with_h0=with_h0, **case)
    y, hT = gpu_ssd(inp)
    yr, hr = oracle_ssd(inp)
    check("y", y, yr, torch.bfloat16)
    check("hT", hT, hr, torch.bfloat16)


def test_ssd_without_skip_and_bias():
    """D and dt_bias absent: the scan part of y alone (D x no longer masks it)."""
    inp = workloads.make_ssd_inputs(SW[0], dstate=128, seqlen=150)
    inp["D"] = None
    inp["dt_bias"] = None
    y, hT = gpu_ssd(inp)
    yr, hr = oracle_ssd(inp)
    check("y", y, yr, torch.bfloat16)
    check("hT", hT, hr, torch.bfloat16)


def test_ssd_chained_calls():
    """A sequence fed as three calls through the carried state matches the
    oracle's single call."""
    inp = workloads.make_ssd_inputs(SW[0], dstate=128, seqlen=300, with_h0=True)
    yr, hr = oracle_ssd(inp)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    h = d["h0"]
    ys = []
    for a, b in [(0, 70), (70, 192), (192, 300)]:
        sl = slice(a, b)
        y, h = ssm.ssd_fwd(d["x"][:, sl].contiguous(), d["dt"][:, sl].contiguous(), d["A"],
                           d["B"][:, sl].contiguous(), d["C"][:, sl].contiguous(), d["D"], d["dt_bias"], h,
                           return_final_state=True)
        ys.append(y)
    torch.cuda.synchronize()
    check("y chained", torch.cat(ys, dim=1).float().cpu().double().numpy(), yr, torch.bfloat16)
    check("hT chained", h.cpu().double().numpy(), hr, torch.bfloat16)


def test_ssd_empty_sequence_passes_state():
    inp = workloads.make_ssd_inputs(SW[0], dstate=64, seqlen=0, with_h0=True)
    y, hT = gpu_ssd(inp)
    assert y.shape[1] == 0
    assert np.array_equal(hT, inp["h0"].double().numpy())


def test_ssd_deterministic():
    inp = workloads.make_ssd_inputs(SW[0], dstate=128, seqlen=200)
    y1, h1 = gpu_ssd(inp)
    y2, h2 = gpu_ssd(inp)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


def test_ssd_mamba2_full_size_sampled_heads():
    """The page's Mamba-2 layer shape at B4 L8192 (H64 P64 N128), launched as the
    bench launches it; heads are independent, so two heads of every batch row are
    checked against the oracle (their group's B and C)."""
    w = SW[1]
    inp = workloads.make_ssd_inputs(w)
    y, hT = gpu_ssd(inp)
    for hsel in (0, 37):
        sub = {k: v for k, v in inp.items()}
        hi = torch.tensor([hsel])
        for k in ("x", "dt"):
            sub[k] = inp[k].index_select(2, hi).contiguous()
        for k in ("A", "D", "dt_bias"):
            sub[k] = inp[k].index_select(0, hi)
        yr, hr = oracle.ssd(sub["x"], sub["dt"], sub["A"], inp["B"], inp["C"], D=sub["D"], dt_bias=sub["dt_bias"])
        check(f"y head {hsel}", y[:, :, hsel:hsel + 1], yr, torch.bfloat16)
        check(f"hT head {hsel}", hT[:, hsel:hsel + 1], hr, torch.bfloat16)


def _planned_splits(d, time_splits):
    """Segments the library runs for these device inputs (with the workspace it asks for)."""
    y = torch.empty_like(d["x"])  # held until the plan is taken: the workspace must not reuse its memory
    a = ssm.make_ssd_args(*(d[k] for k in TENS), y=y, time_splits=time_splits)
    ws = torch.empty(max(ssm.ssd_workspace_bytes(a), 1), dtype=torch.uint8, device=DEV)
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    return ssm.ssd_plan(a)


# (shape, asked segments, segments run): ragged last chunks, one chunk per
# segment, a last segment of one token
SPLIT_CASES = [
    (dict(batch=2, nheads=4, ngroups=2, dstate=64, seqlen=64 * 13 + 17), 3, 3),
    (dict(batch=1, nheads=2, ngroups=1, dstate=128, seqlen=64 * 9), 9, 9),
    (dict(batch=1, nheads=2, ngroups=1, dstate=256, seqlen=64 * 8 + 1), 9, 9),
    (dict(batch=2, nheads=4, ngroups=2, dstate=128, seqlen=64 * 20 + 5), 7, 7),
    (dict(batch=1, nheads=3, ngroups=1, dstate=64, seqlen=64 * 10), 4, 4),  # 10 chunks: 3, 3, 3, 1
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[f"N{c[0]['dstate']}-L{c[0]['seqlen']}-S{c[1]}" for c in SPLIT_CASES])
@pytest.mark.parametrize("with_h0", [False, True], ids=["zero-state", "h0"])
def test_ssd_time_split_all_elements(case, with_h0):
    """Time segments (state-only pass, then the full pass folding the summaries)
    against the oracle on every element of y and the final state."""
    shape, asked, runs = case
    inp = workloads.make_ssd_inputs(SW[0], with_h0=with_h0, seed_extra=(31,), **shape)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    assert _planned_splits(d, asked) == runs
    y, hT = ssm.ssd_fwd(*(d[k] for k in TENS), return_final_state=True, time_splits=asked)
    torch.cuda.synchronize()
    yr, hr = oracle_ssd(inp)
    check("y", y.float().cpu().double().numpy(), yr, torch.bfloat16)
    check("hT", hT.cpu().double().numpy(), hr, torch.bfloat16)


def test_ssd_time_split_reuses_workspace():
    """Two split calls in a row through one workspace, the second shorter: the
    summaries of the first leave nothing behind."""
    big = workloads.make_ssd_inputs(SW[0], batch=1, nheads=2, ngroups=1, dstate=128, seqlen=64 * 12, seed_extra=(32,))
    small = workloads.make_ssd_inputs(SW[0], batch=1, nheads=2, ngroups=1, dstate=128, seqlen=64 * 5 + 9,
                                      with_h0=True, seed_extra=(33,))
    db = {k: (v.to(DEV) if v is not None else None) for k, v in big.items()}
    ds = {k: (v.to(DEV) if v is not None else None) for k, v in small.items()}
    y1 = torch.empty_like(db["x"])
    a = ssm.make_ssd_args(*(db[k] for k in TENS), y=y1, time_splits=6)
    ws = torch.empty(ssm.ssd_workspace_bytes(a), dtype=torch.uint8, device=DEV)
    y1, h1 = ssm.ssd_fwd(*(db[k] for k in TENS), return_final_state=True, time_splits=6, workspace=ws, out=y1)
    y2, h2 = ssm.ssd_fwd(*(ds[k] for k in TENS), return_final_state=True, time_splits=3, workspace=ws)
    torch.cuda.synchronize()
    for (y, h), inp in (((y1, h1), big), ((y2, h2), small)):
        yr, hr = oracle_ssd(inp)
        check("y", y.float().cpu().double().numpy(), yr, torch.bfloat16)
        check("hT", h.cpu().double().numpy(), hr, torch.bfloat16)


def test_ssd_longctx_full_size_sampled_heads():
    """One sequence of 32768 tokens (B1 H64 P64 N128): 64 (b, h) pairs, so the
    library cuts it into 4 time segments; as the bench launches it.  Three heads
    checked against the oracle on every token."""
    w = workloads.SSD_BY_NAME["mamba2_longctx_B1_L32768_H64_P64_N128"]
    inp = workloads.make_ssd_inputs(w, with_h0=True)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    assert _planned_splits(d, 0) == 4
    y, hT = ssm.ssd_fwd(*(d[k] for k in TENS), return_final_state=True)
    torch.cuda.synchronize()
    y, hT = y.float().cpu().double().numpy(), hT.cpu().double().numpy()
    for hsel in (0, 37, 63):
        hi = torch.tensor([hsel])
        yr, hr = oracle.ssd(inp["x"].index_select(2, hi).contiguous(), inp["dt"].index_select(2, hi).contiguous(),
                            inp["A"].index_select(0, hi), inp["B"], inp["C"], D=inp["D"].index_select(0, hi),
                            dt_bias=inp["dt_bias"].index_select(0, hi), s0=inp["h0"].index_select(1, hi))
        check(f"y head {hsel}", y[:, :, hsel:hsel + 1], yr, torch.bfloat16)
        check(f"hT head {hsel}", hT[:, hsel:hsel + 1], hr, torch.bfloat16)


def test_ssd_time_split_state_only_sub_segments():
    """Segments of 16 chunks whose state-only pass runs in sub-segments of 4
    (the planner's choice for B1 H2 with 3 segments): every element."""
    inp = workloads.make_ssd_inputs(SW[0], batch=1, nheads=2, ngroups=1, dstate=128, seqlen=64 * 48 - 13,
                                    with_h0=True, seed_extra=(35,))
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    assert _planned_splits(d, 3) == 3
    y, hT = ssm.ssd_fwd(*(d[k] for k in TENS), return_final_state=True, time_splits=3)
    torch.cuda.synchronize()
    yr, hr = oracle_ssd(inp)
    check("y", y.float().cpu().double().numpy(), yr, torch.bfloat16)
    check("hT", hT.cpu().double().numpy(), hr, torch.bfloat16)
