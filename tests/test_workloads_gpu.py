"""The five workloads at full size, launched exactly as bench.py launches them,
checked against the fp64 oracle on sampled channels (chains are independent,
so a channel's outputs depend only on that channel's inputs and B, C)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mamba_selective_scan_06_amd as ssm
import workloads
from tests.gpu_helpers import check, gpu_scan, oracle_scan, sample_channels, select, to_dev

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP GPU"),
]

W = workloads.WORKLOADS


def test_w0_tiny_fp32_all_elements():
    w = W[0]
    inp = workloads.make_inputs(w)
    y, hT = gpu_scan(to_dev(inp))
    yr, hr = oracle_scan(inp)
    check("y", y, yr, w.dtype)
    check("hT", hT, hr, w.dtype)


@pytest.mark.parametrize("wi", [1, 2])
def test_layer_scan_sampled(wi):
    w = W[wi]
    inp = workloads.make_inputs(w)
    y, hT = gpu_scan(to_dev(inp))
    didx = sample_channels(w.dim, k=40, seed=wi)
    bidx = list(range(w.batch))
    sub = select(inp, bidx, didx)
    yr, hr = oracle_scan(sub)
    check("y", y[np.ix_(bidx, range(w.seqlen), didx)], yr, w.dtype)
    check("hT", hT[np.ix_(bidx, didx)], hr, w.dtype)


def run_chunked(d, chunks):
    """The long sequence as `chunks` calls, hT of one call feeding h0 of the next."""
    L = d["x"].shape[1]
    step = L // chunks
    h = torch.zeros(d["x"].shape[0], d["x"].shape[2], d["A"].shape[1], device=d["x"].device)
    h_next = torch.empty_like(h)
    y = torch.empty_like(d["x"])
    for k in range(chunks):
        sl = slice(k * step, (k + 1) * step)
        ssm.scan_fwd(d["x"][:, sl], d["delta"][:, sl], d["A"], d["B"][:, sl], d["C"][:, sl], d["D"],
                     d["z"][:, sl], d["delta_bias"], h, out=y[:, sl], final_state_out=h_next)
        h, h_next = h_next, h
    return y, h


def test_w3_long_context_chunked():
    w = W[3]
    inp = workloads.make_inputs(w)
    d = to_dev(inp)
    y, h = run_chunked(d, w.chunks)
    didx = sample_channels(w.dim, k=12, seed=3)
    di = torch.tensor(didx, device=y.device)
    torch.cuda.synchronize()
    sub = select(inp, [0], didx)
    yr, hr = oracle_scan(sub)
    ys = y.index_select(2, di).float().cpu().double().numpy()
    check("y chunked", ys, yr, w.dtype)
    check("hT chunked", h.index_select(1, di).cpu().double().numpy(), hr, w.dtype)
    # one call over the whole sequence (time-split inside the call)
    y1, h1 = ssm.scan_fwd(d["x"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["delta_bias"],
                          None, return_final_state=True)
    torch.cuda.synchronize()
    check("y single call", y1.index_select(2, di).float().cpu().double().numpy(), yr, w.dtype)
    check("hT single call", h1.index_select(1, di).cpu().double().numpy(), hr, w.dtype)
    same = torch.equal(y1, y) and torch.equal(h1, h)
    ydiff = float((y1.float() - y.float()).abs().max())
    hdiff = workloads.rel_err(h.cpu().double().numpy(), h1.cpu().double().numpy())
    print(f"  chunked vs single call: bitwise_equal={same} max|dy|={ydiff:.3e} hT rel={hdiff:.3e}")
    assert hdiff <= 1e-4


def test_w4_decode_steps_sampled():
    w = W[4]
    params = workloads.make_inputs(w, seqlen=1)  # A, D, bias, h0
    dp = to_dev(params)
    h = dp["h0"].clone()
    bidx = [0, 1, 77, 128, 254, 255]
    didx = sample_channels(w.dim, k=24, seed=4)
    ys, steps = [], []
    for s in range(w.steps):
        st = workloads.make_decode_step(w, s)
        ds = to_dev(st)
        yt, _ = ssm.scan_fwd(ds["x"], ds["delta"], dp["A"], ds["B"], ds["C"], dp["D"], ds["z"],
                             dp["delta_bias"], h, final_state_out=h)
        ys.append(yt[bidx][:, :, didx].float().cpu())
        steps.append(st)
    torch.cuda.synchronize()
    y = torch.cat(ys, dim=1).double().numpy()
    # the oracle over the same tokens as one L=128 scan of the sampled chains
    seq = {k: torch.cat([st[k] for st in steps], dim=1) for k in ("x", "delta", "B", "C", "z")}
    seq.update({k: params[k] for k in ("A", "D", "delta_bias", "h0")})
    sub = select(seq, bidx, didx)
    yr, hr = oracle_scan(sub)
    check("y", y, yr, w.dtype)
    check("hT", h.cpu().double().numpy()[np.ix_(bidx, didx)], hr, w.dtype)
