"""Checkpoints: the forward (ssm_scan_fwd with `checkpoints`) writes the state
after every T-th token, and the backward (ssm_scan_bwd with the same
checkpoints) starts each chunk from them instead of running the forward
recurrence again.

- Forward: entry i must be the oracle's final state over the first (i + 1) T
  tokens (same inputs, same h0), to the forward's own tolerance
  (workloads.rel_err), and y and hT must be bitwise those of the same call
  without checkpoints (the saving kernel shares every arithmetic step).
- Backward: every gradient against the oracle's, to the backward's tolerance,
  for each kernel family and discretisation that writes checkpoints
  (NSPLIT structured and generic decays, the zero-order hold, time-split
  forwards, LANE, N <= 4 with 16-token chunks), and at full size.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mamba_selective_scan_06_amd as ssm
import oracle
import workloads
from tests.gpu_helpers import DEV, ORACLE_THREADS, check, sample_channels, select, to_dev

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP GPU"),
]

W = workloads.WORKLOADS
TENSORS = ("x", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")


def _case(wi, *, with_h0=True, seed=0, A=None, **shape):
    w = W[wi]
    inp = workloads.make_inputs(w, seed_extra=(71, seed), **shape)
    x = inp["x"]
    cot = workloads.make_cotangents(w, batch=x.shape[0], seqlen=x.shape[1], dim=x.shape[2],
                                    dstate=inp["A"].shape[1], seed_extra=(71, seed))
    if with_h0 and inp["h0"] is None:
        inp["h0"] = 0.5 * cot["dhT"].flip(0).contiguous()
    if A is not None:
        inp["A"] = A
    return w, inp, cot


def gpu_fwd(d, **kw):
    """y, hT and the checkpoints of one forward call."""
    x, A = d["x"], d["A"]
    ck = torch.full(ssm.checkpoint_shape(x.shape[0], x.shape[1], x.shape[2], A.shape[1]), float("nan"),
                    dtype=torch.float32, device=DEV)
    y, hT = ssm.scan_fwd(*(d.get(k) for k in TENSORS), return_final_state=True, checkpoints=ck, **kw)
    y0, h0 = ssm.scan_fwd(*(d.get(k) for k in TENSORS), return_final_state=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(hT, h0), "saving checkpoints changed y or hT"
    return y, hT, ck


def oracle_prefix_states(inp, T, entries, zoh=False):
    """The oracle's state after (i + 1) T tokens, i < entries: (B, entries, D, N)."""
    out = []
    for i in range(entries):
        p = (i + 1) * T
        sub = dict(inp)
        for k in ("x", "delta", "z", "B", "C"):
            if sub[k] is not None:
                sub[k] = inp[k][:, :p].contiguous()
        _, hT = oracle.scan(*(sub.get(k) for k in TENSORS), zoh=zoh, threads=ORACLE_THREADS)
        out.append(hT)
    return np.stack(out, axis=1)


FWD_CASES = {
    "nsplit-struct-bf16": (1, dict(batch=2, seqlen=203, dim=130), {}),
    "nsplit-generic-f32": (0, dict(seqlen=150, dim=70), dict(generic_a=True)),
    "nsplit-zoh-struct": (1, dict(batch=2, seqlen=131, dim=64), dict(zoh=True)),
    "nsplit-zoh-generic": (0, dict(seqlen=99, dim=64), dict(zoh=True, generic_a=True)),
    "nsplit-time-split": (1, dict(batch=1, seqlen=777, dim=96), dict(time_splits=3)),
    "lane-N12": (0, dict(seqlen=120, dim=40, dstate=12), {}),
    "nsplit-N4-T16": (0, dict(seqlen=150, dim=64, dstate=4), {}),
}


@pytest.mark.parametrize("case", sorted(FWD_CASES))
def test_forward_checkpoints_are_the_oracle_states(case):
    wi, shape, kw = FWD_CASES[case]
    w, inp, _ = _case(wi, **shape)
    d = to_dev(inp)
    y, hT, ck = gpu_fwd(d, **kw)
    N = inp["A"].shape[1]
    T = ssm.checkpoint_tokens(N)
    ref = oracle_prefix_states(inp, T, ck.shape[1], zoh=kw.get("zoh", False))
    check("checkpoints", ssm.checkpoint_states(ck, N).cpu().double().numpy(), ref, w.dtype)
    yr, hr = oracle.scan(*(inp.get(k) for k in TENSORS), zoh=kw.get("zoh", False), threads=ORACLE_THREADS)
    check("y", y.float().cpu().double().numpy(), yr, w.dtype)
    check("hT", hT.cpu().double().numpy(), hr, w.dtype)


BWD_CASES = {
    "w0-full": (0, dict(), {}, {}),
    "w1-ragged": (1, dict(batch=2, seqlen=300, dim=200), {}, {}),
    "w2-reduced": (2, dict(batch=1, seqlen=777, dim=129), {}, {}),
    "generic-f32": (0, dict(batch=2, seqlen=157, dim=96), dict(generic_a=True), {}),
    "zoh": (1, dict(batch=2, seqlen=203, dim=130), dict(zoh=True), {}),
    "fwd-split3-bwd-split5": (1, dict(batch=1, seqlen=777, dim=96), dict(time_splits=3), dict(time_splits=5)),
    "bwd-1000-splits": (0, dict(batch=2, seqlen=157, dim=96), {}, dict(time_splits=1000)),
    "lane-N12": (0, dict(seqlen=120, dim=40, dstate=12), {}, {}),
    "N4-T16": (1, dict(batch=2, seqlen=150, dim=64, dstate=4), {}, {}),
    "L-below-one-chunk": (0, dict(seqlen=7, dim=64), {}, {}),
}


@pytest.mark.parametrize("case", sorted(BWD_CASES))
def test_backward_from_checkpoints_all_elements(case):
    wi, shape, fkw, bkw = BWD_CASES[case]
    w, inp, cot = _case(wi, seed=1, **shape)
    d = to_dev(inp)
    _, _, ck = gpu_fwd(d, **fkw)
    zoh = fkw.get("zoh", False)
    g = ssm.scan_bwd(*(d.get(k) for k in TENSORS), dy=cot["dy"].to(DEV), dhT=cot["dhT"].to(DEV), checkpoints=ck,
                     generic_a=fkw.get("generic_a", False), zoh=zoh, **bkw)
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(*(inp.get(k) for k in TENSORS), dy=cot["dy"], dhT=cot["dhT"], zoh=zoh)
    for k in sorted(ref):
        check("d" + k, g[k].float().cpu().double().numpy(), ref[k], w.dtype)


def test_backward_from_checkpoints_deterministic_and_workspace_reuse():
    """Two calls through one workspace give bitwise the same gradients."""
    w, inp, cot = _case(1, seed=2, batch=2, seqlen=256, dim=160)
    d = to_dev(inp)
    _, _, ck = gpu_fwd(d)
    dy, dhT = cot["dy"].to(DEV), cot["dhT"].to(DEV)
    a = ssm.make_bwd_args(*(d.get(k) for k in TENSORS), dy=dy, dhT=dhT, checkpoints=ck)
    ws = torch.empty(ssm.bwd_workspace_bytes(a), dtype=torch.uint8, device=DEV)
    g1 = ssm.scan_bwd(*(d.get(k) for k in TENSORS), dy=dy, dhT=dhT, checkpoints=ck, workspace=ws)
    g2 = ssm.scan_bwd(*(d.get(k) for k in TENSORS), dy=dy, dhT=dhT, checkpoints=ck, workspace=ws)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_full_size_forward_and_backward_from_checkpoints():
    """The 1.4B-shaped layer (B4 L8192 D4096 N16 bf16): forward writing
    checkpoints, then the backward from them, as the bench runs the pair.
    Checkpoints of sampled channels against the oracle's prefix states at
    eight positions; per-channel gradients on sampled channels of every batch
    row; dB and dC of batch row 0 in full."""
    w, inp, cot = _case(2, seed=3)
    d = to_dev(inp)
    x, A = d["x"], d["A"]
    ck = torch.empty(ssm.checkpoint_shape(*x.shape, A.shape[1]), dtype=torch.float32, device=DEV)
    ssm.scan_fwd(*(d.get(k) for k in TENSORS), checkpoints=ck)
    g = ssm.scan_bwd(*(d.get(k) for k in TENSORS), dy=cot["dy"].to(DEV), dhT=cot["dhT"].to(DEV), checkpoints=ck)
    torch.cuda.synchronize()
    del d
    g = {k: v.float().cpu().double().numpy() for k, v in g.items()}
    didx = sample_channels(w.dim, k=12, seed=24)
    bidx = list(range(w.batch))
    sub = select(inp, bidx, didx)
    # checkpoints at eight positions spread over the row
    for i in (0, 1, 127, 128, 511, 700, 1000, ck.shape[1] - 1):
        p = (i + 1) * 8
        pre = {k: (v[:, :p].contiguous() if k in ("x", "delta", "z", "B", "C") and v is not None else v)
               for k, v in sub.items()}
        _, hr = oracle.scan(*(pre.get(k) for k in TENSORS), threads=ORACLE_THREADS)
        got = ssm.checkpoint_states(ck[:, i:i + 1], w.dstate)[:, 0]
        got = got.index_select(1, torch.tensor(didx, device=ck.device)).cpu().double().numpy()
        check(f"checkpoint {i}", got, hr, w.dtype)
    ref = oracle.scan_bwd(*(sub.get(k) for k in TENSORS), dy=cot["dy"].index_select(2, torch.tensor(didx)),
                          dhT=cot["dhT"].index_select(1, torch.tensor(didx)))
    ix = np.ix_(bidx, range(w.seqlen), didx)
    for k in ("x", "delta", "z"):
        check("d" + k, g[k][ix], ref[k], w.dtype)
    check("dA", g["A"][didx], ref["A"], w.dtype)
    for k in ("D", "delta_bias"):
        check("d" + k, g[k][didx], ref[k], w.dtype)
    check("dh0", g["h0"][np.ix_(bidx, didx)], ref["h0"], w.dtype)
    row0 = select(inp, [0], list(range(w.dim)))
    ref0 = oracle.scan_bwd(*(row0.get(k) for k in TENSORS), dy=cot["dy"][:1], dhT=cot["dhT"][:1])
    check("dB row 0", g["B"][:1], ref0["B"], w.dtype)
    check("dC row 0", g["C"][:1], ref0["C"], w.dtype)
