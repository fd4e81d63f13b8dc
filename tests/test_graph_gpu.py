"""Decode steps captured in a HIP graph (torch.cuda.CUDAGraph over the C ABI):
every replay must give the eager result bit for bit.

The library allocates nothing and issues no memset inside a call, so a chain of
ssm_scan_fwd decode steps can be captured.  The graph is replayed several
times with the program's own eager work and synchronisations between the
replays, and each replay is checked against the eager chain.
"""
from __future__ import annotations

import pytest
import torch

import mamba_selective_scan_06_amd as ssm
import workloads
from tests.gpu_helpers import DEV, to_dev

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP GPU"),
]


@pytest.mark.parametrize("zoh", [False, True], ids=["euler", "zoh"])
def test_decode_chain_graph_replays_match_eager(zoh):
    w = workloads.WORKLOADS[4]
    B, D, nsteps = 16, 320, 8
    inp = workloads.make_inputs(w, batch=B, seqlen=1, dim=D)
    A, Dsk, bias = (inp[k].to(DEV) for k in ("A", "D", "delta_bias"))
    h0 = inp["h0"].to(DEV)
    steps = []
    for t in range(nsteps):
        st = workloads.make_decode_step(w, t, batch=B, dim=D)
        steps.append({k: (v.to(DEV) if v is not None else None) for k, v in st.items()})
    h = h0.clone()
    ys = [torch.empty_like(steps[0]["x"]) for _ in steps]

    def chain():
        for st, y in zip(steps, ys):
            ssm.scan_fwd(st["x"], st["delta"], A, st["B"], st["C"], Dsk, st["z"], bias, h, out=y,
                         final_state_out=h, zoh=zoh)

    chain()  # eager reference (also the warm-up before capture)
    torch.cuda.synchronize()
    h_ref, y_ref = h.clone(), [y.clone() for y in ys]

    g = torch.cuda.CUDAGraph()
    h.copy_(h0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        chain()
    torch.cuda.synchronize()
    for rep in range(3):
        h.copy_(h0)
        for y in ys:
            y.zero_()
        _ = (torch.randn(1024, device=DEV) * 2).sum().item()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, h_ref), f"replay {rep}: final state differs from the eager chain"
        for t, (y, yr) in enumerate(zip(ys, y_ref)):
            assert torch.equal(y, yr), f"replay {rep}: y of step {t} differs from the eager chain"


def _replays_match_eager(run, reset=lambda: None, reps=3):
    """run() enqueues the calls and returns their output tensors.  Eager result
    first, then capture, then `reps` replays each compared bit for bit."""
    reset()
    ref = [o.clone() for o in run()]
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run()
    torch.cuda.synchronize()
    for rep in range(reps):
        reset()
        for o in outs:
            o.fill_(float("nan"))
        _ = (torch.randn(4096, device=DEV) * 3).sum().item()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"replay {rep}: output {i} differs from the eager result"


SCAN = ("x", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")


@pytest.mark.parametrize("variant,splits,N", [("auto", 3, 16), ("lane", 0, 12)], ids=["nsplit-3-segments", "lane-N12"])
def test_scan_forward_graph(variant, splits, N):
    w = workloads.WORKLOADS[1]
    inp = to_dev(workloads.make_inputs(w, batch=2, seqlen=1000, dim=200, dstate=N))
    inp["h0"] = torch.randn(2, 200, N, device=DEV) * 0.5

    def run():
        y, hT = ssm.scan_fwd(*(inp[k] for k in SCAN), return_final_state=True, variant=variant, time_splits=splits)
        return [y, hT]
    _replays_match_eager(run)


def test_scan_backward_graph():
    w = workloads.WORKLOADS[1]
    inp = to_dev(workloads.make_inputs(w, batch=2, seqlen=700, dim=130))
    cot = workloads.make_cotangents(w, batch=2, seqlen=700, dim=130, dstate=16)
    dy, dhT = cot["dy"].to(DEV), cot["dhT"].to(DEV)

    def run():
        g = ssm.scan_bwd(*(inp[k] for k in SCAN), dy=dy, dhT=dhT)
        return [g[k] for k in sorted(g)]
    _replays_match_eager(run)


def test_ssd_and_gla_graph():
    sd = {k: (v.to(DEV) if v is not None else None) for k, v in
          workloads.make_ssd_inputs(workloads.SSD_WORKLOADS[0], batch=2, seqlen=300, with_h0=True).items()}
    gd = {k: (v.to(DEV) if v is not None else None) for k, v in
          workloads.make_gla_inputs(workloads.GLA_WORKLOADS[0], batch=2, seqlen=300, gated=True, with_h0=True).items()}

    def run():
        y1, h1 = ssm.ssd_fwd(*(sd[k] for k in ("x", "dt", "A", "B", "C", "D", "dt_bias", "h0")),
                             return_final_state=True)
        y2, h2 = ssm.gla_fwd(*(gd[k] for k in ("q", "k", "v", "log_f", "in_gate", "h0")), feature_map=True,
                             return_final_state=True)
        return [y1, h1, y2, h2]
    _replays_match_eager(run)


def test_conv_prologue_graph():
    w = workloads.WORKLOADS[1]
    x = workloads.make_inputs(w, batch=2, seqlen=500, dim=130)["x"].to(DEV)
    prm = {k: v.to(DEV) for k, v in workloads.make_conv_params(w, dim=130, width=4).items()}
    state = x[:, :3].flip(1).contiguous()

    def run():
        u, so = ssm.conv1d_silu(x, prm["weight"], prm["bias"], state, return_state=True)
        return [u, so]
    _replays_match_eager(run)
