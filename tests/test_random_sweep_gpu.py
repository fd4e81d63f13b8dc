"""Seeded sweep of random shapes and options through every entry point, each
compared element by element with the fp64 oracle.

Each case draws its shape and options from its own seeded generator.  The
shapes stay small enough for the oracle to finish in well under a second.
- Forward scan: B, L, D, N in 1..64; fp32 or bf16; gate, skip term, bias and
  initial state each on or off; Euler or zero-order hold; structured or random
  decay rates, or the generic path forced; automatic, LANE or forced time
  segments.
- Backward: the same families of options.
- SSD and gated linear attention: state sizes, groups, heads and lengths.
- conv1d + SiLU prologue: widths 1..4, carried state and bias on or off.
The case's parameters are printed before it runs.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mamba_selective_scan_06_amd as ssm
import oracle
import workloads
from tests.gpu_helpers import DEV, check, to_dev

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP GPU"),
]

W = workloads.WORKLOADS
TENSORS = ("x", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")
NSPLIT_N = (4, 8, 16, 32, 64)


def _scan_case(seed):
    """Shape, options and seeded inputs of one forward or backward case."""
    g = np.random.default_rng([20261203, 77, seed])
    dtype = torch.float32 if g.random() < 0.5 else torch.bfloat16
    N = int(g.choice([1, 2, 3, 4, 5, 8, 12, 16, 16, 16, 24, 32, 48, 64]))
    bsz = int(g.integers(1, 5))
    L = int(g.integers(1, 700))
    dim = int(g.integers(1, 300))
    while bsz * L * dim * N > 6_000_000:
        L = max(1, L // 2)
    opts = dict(gate=g.random() < 0.6, skip=g.random() < 0.7, bias=g.random() < 0.8, h0=g.random() < 0.5,
                zoh=g.random() < 0.3, decay=str(g.choice(["structured", "random", "generic"])),
                variant=str(g.choice(["auto", "auto", "lane"])), splits=int(g.choice([0, 0, 2, 3])))
    if N not in NSPLIT_N or opts["variant"] == "lane" or L < 2 * opts["splits"]:
        opts["splits"] = 0
    w = W[0] if dtype == torch.float32 else W[1]
    inp = workloads.make_inputs(w, batch=bsz, seqlen=L, dim=dim, dstate=N, seed_extra=(77, seed))
    if opts["gate"] and inp["z"] is None:
        inp["z"] = torch.from_numpy(g.standard_normal((bsz, L, dim)).astype(np.float32)).to(dtype)
    if not opts["gate"]:
        inp["z"] = None
    if not opts["skip"]:
        inp["D"] = None
    if not opts["bias"]:
        inp["delta_bias"] = None
    inp["h0"] = torch.from_numpy(g.normal(0, 0.5, (bsz, dim, N)).astype(np.float32)) if opts["h0"] else None
    if opts["decay"] == "random":
        inp["A"] = torch.from_numpy(-np.exp(g.normal(0.0, 1.0, (dim, N))).astype(np.float32))
    desc = f"seed={seed} {str(dtype)[6:]} B{bsz} L{L} D{dim} N{N} " + " ".join(f"{k}={v}" for k, v in opts.items())
    return w, inp, opts, desc


@pytest.mark.parametrize("seed", range(40))
def test_random_scan_forward(seed):
    w, inp, o, desc = _scan_case(seed)
    print(" ", desc, flush=True)
    d = to_dev(inp)
    y, hT = ssm.scan_fwd(*(d.get(k) for k in TENSORS), return_final_state=True, zoh=o["zoh"],
                         generic_a=o["decay"] == "generic", variant=o["variant"], time_splits=o["splits"])
    torch.cuda.synchronize()
    yr, hr = oracle.scan(*(inp.get(k) for k in TENSORS), zoh=o["zoh"])
    check("y", y.float().cpu().double().numpy(), yr, w.dtype)
    check("hT", hT.cpu().double().numpy(), hr, w.dtype)


@pytest.mark.parametrize("seed", range(16))
def test_random_scan_backward(seed):
    w, inp, o, desc = _scan_case(1000 + seed)
    print(" ", desc, "(Euler, backward)", flush=True)
    x = inp["x"]
    cot = workloads.make_cotangents(w, batch=x.shape[0], seqlen=x.shape[1], dim=x.shape[2],
                                    dstate=inp["A"].shape[1], seed_extra=(77, seed))
    dhT = cot["dhT"] if o["h0"] else None
    d = to_dev(inp)
    got = ssm.scan_bwd(*(d.get(k) for k in TENSORS), dy=cot["dy"].to(DEV),
                       dhT=None if dhT is None else dhT.to(DEV), generic_a=o["decay"] == "generic")
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(*(inp.get(k) for k in TENSORS), dy=cot["dy"], dhT=dhT)
    for k in sorted(ref):
        check("d" + k, got[k].float().cpu().double().numpy(), ref[k], w.dtype)


def _heads_case(seed):
    g = np.random.default_rng([20261203, 78, seed])
    N = int(g.choice([64, 128, 256]))
    G = int(g.choice([1, 2, 4]))
    H = G * int(g.integers(1, 4))
    return dict(batch=int(g.integers(1, 3)), seqlen=int(g.integers(1, 300)), nheads=H, ngroups=G, dstate=N), g


@pytest.mark.parametrize("seed", range(12))
def test_random_ssd(seed):
    shape, g = _heads_case(seed)
    with_h0 = bool(g.random() < 0.5)
    print(f"  seed={seed} {shape} h0={with_h0}", flush=True)
    inp = workloads.make_ssd_inputs(workloads.SSD_WORKLOADS[0], with_h0=with_h0, seed_extra=(78, seed), **shape)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    y, hT = ssm.ssd_fwd(*(d[k] for k in ("x", "dt", "A", "B", "C", "D", "dt_bias", "h0")), return_final_state=True)
    torch.cuda.synchronize()
    yr, hr = oracle.ssd(*(inp[k] for k in ("x", "dt", "A", "B", "C")), D=inp["D"], dt_bias=inp["dt_bias"],
                        s0=inp["h0"])
    check("y", y.float().cpu().double().numpy(), yr, torch.bfloat16)
    check("hT", hT.cpu().double().numpy(), hr, torch.bfloat16)


@pytest.mark.parametrize("seed", range(12))
def test_random_gla(seed):
    shape, g = _heads_case(100 + seed)
    gated, with_h0, fm = bool(g.random() < 0.7), bool(g.random() < 0.5), bool(g.random() < 0.4)
    print(f"  seed={seed} {shape} gated={gated} h0={with_h0} elu={fm}", flush=True)
    inp = workloads.make_gla_inputs(workloads.GLA_WORKLOADS[0], gated=gated, with_h0=with_h0,
                                    seed_extra=(79, seed), **shape)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    y, hT = ssm.gla_fwd(*(d[k] for k in ("q", "k", "v", "log_f", "in_gate", "h0")), feature_map=fm,
                        return_final_state=True)
    torch.cuda.synchronize()
    yr, hr = oracle.gla(inp["q"], inp["k"], inp["v"], log_f=inp["log_f"], in_gate=inp["in_gate"], s0=inp["h0"],
                        feature_map=fm)
    check("y", y.float().cpu().double().numpy(), yr, torch.bfloat16)
    check("hT", hT.cpu().double().numpy(), hr, torch.bfloat16)


@pytest.mark.parametrize("seed", range(12))
def test_random_conv_prologue(seed):
    g = np.random.default_rng([20261203, 80, seed])
    dtype = torch.float32 if g.random() < 0.5 else torch.bfloat16
    w = W[0] if dtype == torch.float32 else W[1]
    bsz, L, dim, width = int(g.integers(1, 5)), int(g.integers(1, 600)), int(g.integers(1, 300)), int(g.integers(1, 5))
    with_state, with_bias = bool(g.random() < 0.5), bool(g.random() < 0.7)
    print(f"  seed={seed} {str(dtype)[6:]} B{bsz} L{L} D{dim} W{width} state={with_state} bias={with_bias}", flush=True)
    x = workloads.make_inputs(w, batch=bsz, seqlen=L, dim=dim, seed_extra=(80, seed))["x"]
    prm = workloads.make_conv_params(w, dim=dim, width=width, seed_extra=(80, seed))
    bias = prm["bias"] if with_bias else None
    state = None
    if with_state:
        prev = workloads.make_inputs(w, batch=bsz, seqlen=max(width - 1, 1), dim=dim, seed_extra=(80, seed, 1))["x"]
        state = prev[:, :width - 1].contiguous()
    dv = lambda t: None if t is None else t.to(DEV)
    u, so = ssm.conv1d_silu(dv(x), dv(prm["weight"]), dv(bias), dv(state), return_state=True)
    torch.cuda.synchronize()
    ur, _, _ = oracle.conv1d_silu(x, prm["weight"], bias, state)
    check("u", u.float().cpu().double().numpy(), ur, dtype)
    # the carried state is the last W-1 input rows, earlier rows coming from `state`
    full = torch.cat([state if state is not None else torch.zeros(bsz, width - 1, dim, dtype=dtype), x], dim=1)
    assert torch.equal(so.cpu(), full[:, full.shape[1] - (width - 1):, :]), "state_out is not the last W-1 input rows"
