"""Backward scan on the GPU (ssm_scan_bwd through the C ABI) against the fp64
oracle's reverse-mode gradients, on the same seeded inputs and cotangents.

Tolerance: the forward's floored max relative error (workloads.rel_err),
1e-4 for fp32 inputs and 2e-2 for bf16 inputs, applied to every gradient
tensor.  The gradients are fp32 sums of the same kind of terms as the forward
(products of decays, inputs and cotangents accumulated over tokens, channels
or batch rows), and the bf16 outputs carry one bf16 rounding (2^-9).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mamba_selective_scan_06_amd as ssm
import oracle
import workloads
from tests.gpu_helpers import DEV, check, sample_channels, select, to_dev

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP GPU"),
]

W = workloads.WORKLOADS
TENSORS = ("x", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")


def gpu_bwd(dinp, dy, dhT, **kw):
    g = ssm.scan_bwd(*(dinp.get(k) for k in TENSORS), dy=dy, dhT=dhT, **kw)
    torch.cuda.synchronize()
    return {k: v.float().cpu().double().numpy() for k, v in g.items()}


def oracle_bwd(inp, dy, dhT):
    return oracle.scan_bwd(*(inp.get(k) for k in TENSORS), dy=dy, dhT=dhT)


def check_all(got, ref, dtype, keys=None):
    keys = keys or sorted(ref)
    assert set(keys) <= set(got), (sorted(got), keys)
    for k in keys:
        check("d" + k, got[k], ref[k], dtype)


def _case(wi, drop=(), with_h0=False, seed_extra=(), **shape):
    w = W[wi]
    inp = workloads.make_inputs(w, seed_extra=seed_extra, **shape)
    for k in drop:
        inp[k] = None
    x = inp["x"]
    cot = workloads.make_cotangents(w, batch=x.shape[0], seqlen=x.shape[1], dim=x.shape[2],
                                    dstate=inp["A"].shape[1], seed_extra=seed_extra)
    if with_h0 and inp["h0"] is None:
        inp["h0"] = 0.5 * cot["dhT"].flip(0).contiguous()
    return w, inp, cot


# ------------------------------------------------- reduced sizes, every element
SMALL = [
    (0, dict()),                                    # tiny fp32 workload at full size
    (0, dict(seqlen=203, dim=130)),                 # ragged L (chunk 8) and D (32 channels per wave)
    (1, dict(batch=2, seqlen=300, dim=200)),
    (2, dict(batch=1, seqlen=777, dim=129)),
]
OPTS = {
    "full": dict(),
    "h0-dhT": dict(with_h0=True),
    "noD-nogate-nobias": dict(drop=("D", "z", "delta_bias")),
}


@pytest.mark.parametrize("wi,shape", SMALL, ids=[f"w{w}-{'-'.join(f'{k}{v}' for k, v in s.items()) or 'full'}"
                                                 for w, s in SMALL])
@pytest.mark.parametrize("opt", sorted(OPTS))
def test_bwd_small_all_elements(wi, shape, opt):
    o = OPTS[opt]
    w, inp, cot = _case(wi, drop=o.get("drop", ()), with_h0=o.get("with_h0", False), **shape)
    dhT = cot["dhT"] if opt != "full" else None
    got = gpu_bwd(to_dev(inp), cot["dy"].to(DEV), None if dhT is None else dhT.to(DEV))
    ref = oracle_bwd(inp, cot["dy"], dhT)
    check_all(got, ref, w.dtype)


@pytest.mark.parametrize("N", [1, 3, 4, 5, 8, 12, 16, 24, 32, 48, 64])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_bwd_state_sizes(N, dtype):
    """Every lane layout: K = 4 or 8 states per lane, 1, 2, 4 or 8 lanes per
    channel, with and without missing states in the last lane."""
    wi = 0 if dtype == torch.float32 else 1
    w, inp, cot = _case(wi, with_h0=True, batch=2, seqlen=150, dim=70, dstate=N)
    g = torch.Generator().manual_seed(N)
    inp["A"] = -torch.rand(70, N, generator=g) * 3 - 0.05  # unstructured decay rates
    got = gpu_bwd(to_dev(inp), cot["dy"].to(DEV), cot["dhT"].to(DEV))
    ref = oracle_bwd(inp, cot["dy"], cot["dhT"])
    check_all(got, ref, w.dtype)


@pytest.mark.parametrize("splits", [1, 2, 5, 19, 1000])
def test_bwd_time_splits(splits):
    """Segments run from a zero start and are fixed up; any split count gives
    the oracle's gradients (1000 requests: one 8-token chunk per segment)."""
    w, inp, cot = _case(0, with_h0=True, batch=2, seqlen=157, dim=96)
    dinp = to_dev(inp)
    got = gpu_bwd(dinp, cot["dy"].to(DEV), cot["dhT"].to(DEV), time_splits=splits)
    ref = oracle_bwd(inp, cot["dy"], cot["dhT"])
    check_all(got, ref, w.dtype)


@pytest.mark.parametrize("N", [4, 16, 32])
def test_bwd_structured_and_generic_decay(N):
    """A = -(1..N) takes the structured-decay path (powers of one decay); the
    generic flag forces one exp per state.  Both match the oracle."""
    w, inp, cot = _case(1, with_h0=True, batch=2, seqlen=130, dim=96, dstate=N)
    d = to_dev(inp)
    ref = oracle_bwd(inp, cot["dy"], cot["dhT"])
    for generic in (False, True):
        got = gpu_bwd(d, cot["dy"].to(DEV), cot["dhT"].to(DEV), generic_a=generic)
        check_all(got, ref, w.dtype)


def test_bwd_wanted_subset_and_determinism():
    w, inp, cot = _case(1, with_h0=True, batch=2, seqlen=256, dim=160)
    d = to_dev(inp)
    dy, dhT = cot["dy"].to(DEV), cot["dhT"].to(DEV)
    full1 = ssm.scan_bwd(*(d.get(k) for k in TENSORS), dy=dy, dhT=dhT)
    full2 = ssm.scan_bwd(*(d.get(k) for k in TENSORS), dy=dy, dhT=dhT)
    only_x = ssm.scan_bwd(*(d.get(k) for k in TENSORS), dy=dy, dhT=dhT, wanted=("x", "A"))
    torch.cuda.synchronize()
    for k in full1:
        assert torch.equal(full1[k], full2[k]), f"d{k} differs between two identical calls"
    assert set(only_x) == {"x", "A"}
    assert torch.equal(only_x["x"], full1["x"]) and torch.equal(only_x["A"], full1["A"])


def test_bwd_extreme_step_sizes():
    """Raw step sizes far out on both sides of softplus (delta -> 0 and delta ~ raw)."""
    w, inp, cot = _case(0, with_h0=True, batch=1, seqlen=120, dim=64)
    g = torch.Generator().manual_seed(7)
    inp["delta"] = (torch.randn(1, 120, 64, generator=g) * 12.0).float()
    got = gpu_bwd(to_dev(inp), cot["dy"].to(DEV), cot["dhT"].to(DEV))
    ref = oracle_bwd(inp, cot["dy"], cot["dhT"])
    check_all(got, ref, w.dtype)


def test_bwd_empty_problems():
    f32 = torch.float32
    N = 16
    # L == 0: the state passes through, dh0 = dhT; sums over tokens are zero
    A = -torch.ones(8, N, device=DEV)
    x = torch.empty(2, 0, 8, device=DEV)
    Bm = torch.empty(2, 0, N, device=DEV)
    dhT = torch.randn(2, 8, N, device=DEV)
    D = torch.ones(8, device=DEV)
    bias = torch.zeros(8, device=DEV)
    g = ssm.scan_bwd(x, x, A, Bm, Bm, D, None, bias, None, dy=x, dhT=dhT)
    torch.cuda.synchronize()
    assert torch.equal(g["h0"], dhT)
    for k in ("A", "D", "delta_bias"):
        assert torch.count_nonzero(g[k]) == 0
    g = ssm.scan_bwd(x, x, A, Bm, Bm, dy=x)  # no dhT: dh0 = 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(g["h0"]) == 0
    # B == 0: sums over batch rows are zero
    x = torch.empty(0, 5, 8, device=DEV)
    Bm = torch.empty(0, 5, N, device=DEV)
    g = ssm.scan_bwd(x, x, A, Bm, Bm, D, None, bias, dy=x)
    torch.cuda.synchronize()
    for k in ("A", "D", "delta_bias"):
        assert g[k].shape[0] == 8 and torch.count_nonzero(g[k]) == 0
    # D == 0: sums over channels (dB, dC) are zero
    x = torch.empty(2, 5, 0, device=DEV)
    Bm = torch.randn(2, 5, N, device=DEV, dtype=f32)
    g = ssm.scan_bwd(x, x, torch.empty(0, N, device=DEV), Bm, Bm.clone(), dy=x)
    torch.cuda.synchronize()
    assert torch.count_nonzero(g["B"]) == 0 and torch.count_nonzero(g["C"]) == 0


# ------------------------------------------------- full-size workloads
def test_bwd_w1_full_all_elements():
    """The 130M-shaped layer (B8 L2048 D1536 N16 bf16, gate on) at full size."""
    w, inp, cot = _case(1)
    got = gpu_bwd(to_dev(inp), cot["dy"].to(DEV), cot["dhT"].to(DEV))
    ref = oracle_bwd(inp, cot["dy"], cot["dhT"])
    check_all(got, ref, w.dtype)


def test_bwd_w2_full_sampled():
    """The 1.4B-shaped layer (B4 L8192 D4096 N16 bf16) at full size, launched as
    the bench times it.  Per-channel gradients (dx, ddelta, dz, dA, dD,
    ddelta_bias, dh0) on sampled channels of every batch row; dB and dC, which
    sum over all channels of one batch row, on batch row 0 in full."""
    w, inp, cot = _case(2)
    d = to_dev(inp)
    got = gpu_bwd(d, cot["dy"].to(DEV), cot["dhT"].to(DEV))
    del d
    didx = sample_channels(w.dim, k=24, seed=22)
    bidx = list(range(w.batch))
    sub = select(inp, bidx, didx)
    dsub = cot["dy"].index_select(2, torch.tensor(didx))
    hsub = cot["dhT"].index_select(1, torch.tensor(didx))
    ref = oracle_bwd(sub, dsub, hsub)
    ix = np.ix_(bidx, range(w.seqlen), didx)
    for k in ("x", "delta", "z"):
        check("d" + k, got[k][ix], ref[k], w.dtype)
    check("dA", got["A"][didx], ref["A"], w.dtype)
    for k in ("D", "delta_bias"):
        check("d" + k, got[k][didx], ref[k], w.dtype)
    check("dh0", got["h0"][np.ix_(bidx, didx)], ref["h0"], w.dtype)
    row0 = select(inp, [0], list(range(w.dim)))
    ref0 = oracle_bwd(row0, cot["dy"][:1], cot["dhT"][:1])
    check("dB row 0", got["B"][:1], ref0["B"], w.dtype)
    check("dC row 0", got["C"][:1], ref0["C"], w.dtype)
