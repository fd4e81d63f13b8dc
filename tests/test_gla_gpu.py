"""Gated linear attention / mLSTM recurrence on the GPU (ssm_gla_fwd through the
C ABI, the chunked matrix form of the SSD kernel on bf16 MFMA) against the fp64
oracle's recurrence.

Tolerance: 2e-2 floored max relative error (bf16 inputs, workloads.rel_err), as
for the SSD layer: the kernel rounds three MFMA operands to hi + lo bf16 pairs
and y once to bf16.  With the elu + 1 feature map, phi(q) and phi(k) are also
rounded to bf16 (a relative 2^-9 per element) before the products.
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

GW = workloads.GLA_WORKLOADS
TENS = ("q", "k", "v", "log_f", "in_gate", "h0")


def gpu_gla(inp, feature_map=False):
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    y, hT = ssm.gla_fwd(*(d[k] for k in TENS), feature_map=feature_map, return_final_state=True)
    torch.cuda.synchronize()
    return y.float().cpu().double().numpy(), hT.cpu().double().numpy()


def oracle_gla(inp, feature_map=False):
    return oracle.gla(inp["q"], inp["k"], inp["v"], log_f=inp["log_f"], in_gate=inp["in_gate"], s0=inp["h0"],
                      feature_map=feature_map)


CASES = [
    dict(dstate=64, ngroups=2, seqlen=200),
    dict(dstate=128, ngroups=1, seqlen=200),
    dict(dstate=256, ngroups=4, seqlen=130),
    dict(dstate=128, ngroups=2, seqlen=64),   # exactly one chunk
    dict(dstate=128, ngroups=2, seqlen=65),   # one token into the second chunk
    dict(dstate=64, ngroups=1, seqlen=1),
    dict(dstate=256, ngroups=1, seqlen=63),
]


@pytest.mark.parametrize("case", CASES, ids=[f"N{c['dstate']}-G{c['ngroups']}-L{c['seqlen']}" for c in CASES])
@pytest.mark.parametrize("mode", ["gated", "gated-h0", "linear", "linear-elu", "gated-elu-h0"])
def test_gla_small_all_elements(case, mode):
    inp = workloads.make_gla_inputs(GW[0], gated=mode.startswith("gated"), with_h0=mode.endswith("h0"), **case)
    fm = "elu" in mode
    y, hT = gpu_gla(inp, fm)
    yr, hr = oracle_gla(inp, fm)
    check("y", y, yr, torch.bfloat16)
    check("hT", hT, hr, torch.bfloat16)


def test_gla_one_gate_only():
    """Forget gate without input gate, then input gate without forget gate."""
    base = workloads.make_gla_inputs(GW[0], dstate=128, seqlen=150, with_h0=True)
    for drop in ("in_gate", "log_f"):
        inp = dict(base, **{drop: None})
        y, hT = gpu_gla(inp)
        yr, hr = oracle_gla(inp)
        check(f"y without {drop}", y, yr, torch.bfloat16)
        check(f"hT without {drop}", hT, hr, torch.bfloat16)


def test_gla_chained_calls():
    """A sequence fed as three calls through the carried state matches the
    oracle's single call."""
    inp = workloads.make_gla_inputs(GW[0], dstate=128, seqlen=300, with_h0=True)
    yr, hr = oracle_gla(inp, True)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    h = d["h0"]
    ys = []
    for a, b in [(0, 70), (70, 192), (192, 300)]:
        sl = slice(a, b)
        y, h = ssm.gla_fwd(*(d[k][:, sl].contiguous() for k in ("q", "k", "v", "log_f", "in_gate")), h,
                           feature_map=True, return_final_state=True)
        ys.append(y)
    torch.cuda.synchronize()
    check("y chained", torch.cat(ys, dim=1).float().cpu().double().numpy(), yr, torch.bfloat16)
    check("hT chained", h.cpu().double().numpy(), hr, torch.bfloat16)


def test_gla_matches_ssd_kernel_with_ssd_gates():
    """log f = delta A and in_gate = delta reproduce ssm_ssd_fwd without D."""
    sw = workloads.SSD_WORKLOADS[0]
    inp = workloads.make_ssd_inputs(sw, dstate=128, seqlen=200, with_h0=True)
    delta = torch.nn.functional.softplus(inp["dt"].float() + inp["dt_bias"][None, None, :])
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    y1, h1 = ssm.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], None, d["dt_bias"], d["h0"],
                         return_final_state=True)
    y2, h2 = ssm.gla_fwd(d["C"], d["B"], d["x"], (delta * inp["A"][None, None, :]).to(DEV), delta.to(DEV), d["h0"],
                         return_final_state=True)
    torch.cuda.synchronize()
    # the two differ only in how delta is computed (device softplus vs torch's)
    check("y gla vs ssd", y2.float().cpu().double().numpy(), y1.float().cpu().double().numpy(), torch.bfloat16)
    check("hT gla vs ssd", h2.cpu().double().numpy(), h1.cpu().double().numpy(), torch.bfloat16)


def test_gla_empty_sequence_passes_state():
    inp = workloads.make_gla_inputs(GW[0], dstate=64, seqlen=0, with_h0=True)
    y, hT = gpu_gla(inp)
    assert y.shape[1] == 0
    assert np.array_equal(hT, inp["h0"].double().numpy())


def test_gla_deterministic():
    inp = workloads.make_gla_inputs(GW[0], dstate=128, seqlen=200)
    y1, h1 = gpu_gla(inp, True)
    y2, h2 = gpu_gla(inp, True)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


@pytest.mark.parametrize("wi", [1, 2], ids=["mlstm", "linattn-elu"])
def test_gla_full_size_sampled_heads(wi):
    """B4 L8192 H64 P64 N128 as the bench launches it; heads are independent, so
    two heads of every batch row are checked against the oracle."""
    w = GW[wi]
    inp = workloads.make_gla_inputs(w)
    y, hT = gpu_gla(inp, w.feature_map)
    for hsel in (0, 41):
        hi = torch.tensor([hsel])
        sub = dict(inp, v=inp["v"].index_select(2, hi).contiguous())
        for k in ("log_f", "in_gate"):
            if inp[k] is not None:
                sub[k] = inp[k].index_select(2, hi).contiguous()
        yr, hr = oracle_gla(sub, w.feature_map)
        check(f"y head {hsel}", y[:, :, hsel:hsel + 1], yr, torch.bfloat16)
        check(f"hT head {hsel}", hT[:, hsel:hsel + 1], hr, torch.bfloat16)


@pytest.mark.parametrize("case", [dict(dstate=64, ngroups=2, seqlen=200), dict(dstate=256, ngroups=1, seqlen=130),
                                  dict(dstate=128, ngroups=4, seqlen=1)], ids=["N64-G2", "N256-G1", "N128-L1"])
def test_feature_map_pass_matches_in_kernel_map(case):
    """phi applied once per call into the workspace, or by every head's
    workgroup in its staging: bitwise the same y and state."""
    inp = workloads.make_gla_inputs(GW[0], gated=True, with_h0=True, **case)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    args = [d[k] for k in TENS]
    y1, h1 = ssm.gla_fwd(*args, feature_map=True, return_final_state=True)  # workspace: the pass
    y2, h2 = ssm.gla_fwd(*args, feature_map=True, return_final_state=True,
                         workspace=torch.empty(0, dtype=torch.uint8, device=DEV))  # declined: in the kernel
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    yr, hr = oracle_gla(inp, True)
    check("y", y1.float().cpu().double().numpy(), yr, torch.bfloat16)
    check("hT", h1.cpu().double().numpy(), hr, torch.bfloat16)


def _planned_splits(d, time_splits, feature_map):
    y = torch.empty_like(d["v"])  # held until the plan is taken: the workspace must not reuse its memory
    a = ssm.make_gla_args(*(d[k] for k in TENS), y=y, feature_map=feature_map, time_splits=time_splits)
    ws = torch.empty(max(ssm.gla_workspace_bytes(a), 1), dtype=torch.uint8, device=DEV)
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    return ssm.gla_plan(a)


SPLIT_CASES = [
    (dict(batch=2, nheads=4, ngroups=2, dstate=64, seqlen=64 * 13 + 17), 3),
    (dict(batch=1, nheads=2, ngroups=1, dstate=256, seqlen=64 * 8 + 1), 9),
    (dict(batch=1, nheads=4, ngroups=4, dstate=128, seqlen=64 * 11 + 40), 6),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[f"N{c[0]['dstate']}-L{c[0]['seqlen']}-S{c[1]}" for c in SPLIT_CASES])
@pytest.mark.parametrize("mode", ["gated-h0", "linear", "linear-elu-h0"])
def test_gla_time_split_all_elements(case, mode):
    """Time segments against the oracle on every element; with the feature map
    the summaries sit behind phi(k) and phi(q) in the workspace."""
    shape, asked = case
    inp = workloads.make_gla_inputs(GW[0], gated=mode.startswith("gated"), with_h0=mode.endswith("h0"),
                                    seed_extra=(34,), **shape)
    fm = "elu" in mode
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    assert _planned_splits(d, asked, fm) == asked
    y, hT = ssm.gla_fwd(*(d[k] for k in TENS), feature_map=fm, return_final_state=True, time_splits=asked)
    torch.cuda.synchronize()
    yr, hr = oracle_gla(inp, fm)
    check("y", y.float().cpu().double().numpy(), yr, torch.bfloat16)
    check("hT", hT.cpu().double().numpy(), hr, torch.bfloat16)


def test_gla_longctx_full_size_sampled_heads():
    """mLSTM gates over one 32768-token sequence (B1 H64 P64 N128): 4 time
    segments chosen by the library, as the bench launches it; three heads
    against the oracle."""
    w = workloads.GLA_BY_NAME["mlstm_longctx_B1_L32768_H64_P64_N128"]
    inp = workloads.make_gla_inputs(w, with_h0=True)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    assert _planned_splits(d, 0, w.feature_map) == 4
    y, hT = gpu_gla(inp, w.feature_map)
    for hsel in (0, 41, 63):
        hi = torch.tensor([hsel])
        sub = dict(inp, v=inp["v"].index_select(2, hi).contiguous(), h0=inp["h0"].index_select(1, hi).contiguous())
        for k in ("log_f", "in_gate"):
            sub[k] = inp[k].index_select(2, hi).contiguous()
        yr, hr = oracle_gla(sub, w.feature_map)
        check(f"y head {hsel}", y[:, :, hsel:hsel + 1], yr, torch.bfloat16)
        check(f"hT head {hsel}", hT[:, hsel:hsel + 1], hr, torch.bfloat16)


@pytest.mark.parametrize("mode", ["gated-h0", "linear-elu"])
def test_gla_time_split_state_only_sub_segments(mode):
    """Segments of 16 chunks, state-only sub-segments of 4: every element."""
    inp = workloads.make_gla_inputs(GW[0], batch=1, nheads=2, ngroups=1, dstate=64, seqlen=64 * 48 - 5,
                                    gated=mode.startswith("gated"), with_h0=mode.endswith("h0"), seed_extra=(36,))
    fm = "elu" in mode
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    assert _planned_splits(d, 3, fm) == 3
    y, hT = ssm.gla_fwd(*(d[k] for k in TENS), feature_map=fm, return_final_state=True, time_splits=3)
    torch.cuda.synchronize()
    yr, hr = oracle_gla(inp, fm)
    check("y", y.float().cpu().double().numpy(), yr, torch.bfloat16)
    check("hT", hT.cpu().double().numpy(), hr, torch.bfloat16)
