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
from tests.gpu_helpers import DEV

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
