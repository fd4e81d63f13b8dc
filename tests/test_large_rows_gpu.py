"""Maximum sizes: batch rows of more than 2 and 4 GiB per tensor, in one call.

The main kernel addresses a row through buffer descriptors with 32-bit byte
offsets; its windows move along the row so that offsets stay small whatever
the row length.  These cases put rows past 2^31 and 2^32 bytes through it,
unsplit and with forced time segments that start gigabytes into the row, and
compare sampled channels (each a whole independent chain over every token)
with the fp64 oracle.  Every y must also be finite.

The SSD layer's x and y pass 2 GiB per batch row at L = 262208 (64 heads of
64 channels); three sampled heads are compared, since the heads of a group are
independent given the shared B and C.

The backward cuts such rows into segments whose spans fit its 32-bit offsets.
Its per-channel gradients (dx, ddelta, dz, dA, dD, ddelta_bias, dh0) are
compared on sampled channels.  dB and dC are sums over every channel, out of
the oracle's reach at this size, and are checked to be finite.
"""
from __future__ import annotations

import gc

import numpy as np
import pytest
import torch

import mamba_selective_scan_06_amd as ssm
import workloads
import oracle
from tests.gpu_helpers import DEV, check, oracle_scan, sample_channels, select

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP GPU"),
]

TENS = ("x", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")

CASES = [
    # (workload index for dtype and recipe, B, L, D): D ragged against 64-channel
    # blocks, L ragged against 16-token tiles
    (1, 1, 262_152, 4104),   # bf16: 2.15 GB per row (> 2^31 bytes)
    (0, 1, 270_008, 4104),   # fp32: 4.43 GB per row (> 2^32 bytes)
]


@pytest.mark.parametrize("wi,bsz,L,dim", CASES, ids=["bf16-row2.15GB", "fp32-row4.43GB"])
def test_rows_beyond_32bit_offsets(wi, bsz, L, dim):
    w = workloads.WORKLOADS[wi]
    inp = workloads.make_large_inputs(w, batch=bsz, seqlen=L, dim=dim)
    row_bytes = L * dim * inp["x"].element_size()
    print(f"  B={bsz} L={L} D={dim} {w.dtype}: {row_bytes / 2**30:.2f} GiB per row", flush=True)
    chans = sample_channels(dim, k=12, seed=L)
    sub = select(inp, list(range(bsz)), chans)
    yr, hr = oracle_scan(sub)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    del inp
    gc.collect()
    y = torch.empty_like(d["x"])
    hT = torch.empty((bsz, dim, w.dstate), dtype=torch.float32, device=DEV)
    a = ssm.make_args(d["x"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["delta_bias"], None, hT, y)
    assert ssm.plan(a)[0] == "nsplit"
    # time_splits=1 runs the windowed kernel as one segment over the whole row;
    # 0 lets the planner split (it takes 3 segments here given a workspace)
    a.time_splits = 1
    assert ssm.plan(a) == ("nsplit", 1)
    ci = torch.as_tensor(chans, device=DEV)
    for splits in (1, 0, 4):
        y.fill_(float("nan"))
        ssm.scan_fwd(d["x"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["delta_bias"],
                     out=y, final_state_out=hT, time_splits=splits)
        torch.cuda.synchronize()
        print(f"  time_splits={splits}", flush=True)
        assert bool(torch.isfinite(y).all())
        ys = y.index_select(2, ci).float().cpu().double().numpy()
        hs = hT.index_select(1, ci).cpu().double().numpy()
        check(f"y splits={splits}", ys, yr, w.dtype)
        check(f"hT splits={splits}", hs, hr, w.dtype)
    del d, y, hT
    torch.cuda.empty_cache()


def test_row_beyond_2gib_zoh_generic_decays():
    """The windowed instantiation with the zero-order hold and every decay its
    own exp (random decay rates, generic path forced), as one segment
    (time_splits=1) and in 3 segments."""
    w = workloads.WORKLOADS[1]
    bsz, L, dim = 1, 262_152, 4104
    inp = workloads.make_large_inputs(w, batch=bsz, seqlen=L, dim=dim, seed_extra=(3,))
    inp["A"] = -torch.rand(dim, w.dstate, generator=torch.Generator().manual_seed(3)) * 3 - 0.05
    inp["h0"] = torch.randn(bsz, dim, w.dstate, generator=torch.Generator().manual_seed(4)) * 0.5
    print(f"  ZOH, generic decays: B={bsz} L={L} D={dim} bf16", flush=True)
    chans = sample_channels(dim, k=8, seed=L + 2)
    yr, hr = oracle.scan(*(select(inp, [0], chans).get(k) for k in TENS), zoh=True)
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    del inp
    gc.collect()
    ci = torch.as_tensor(chans, device=DEV)
    for splits in (1, 3):
        y, hT = ssm.scan_fwd(*(d.get(k) for k in TENS), return_final_state=True, zoh=True, generic_a=True,
                             time_splits=splits)
        torch.cuda.synchronize()
        print(f"  time_splits={splits}", flush=True)
        check(f"y splits={splits}", y.index_select(2, ci).float().cpu().double().numpy(), yr, w.dtype)
        check(f"hT splits={splits}", hT.index_select(1, ci).cpu().double().numpy(), hr, w.dtype)
        del y, hT
    del d
    torch.cuda.empty_cache()


def test_backward_row_beyond_2gib():
    w = workloads.WORKLOADS[1]
    bsz, L, dim = 1, 262_152, 4104
    inp = workloads.make_large_inputs(w, batch=bsz, seqlen=L, dim=dim)
    inp["h0"] = torch.randn(bsz, dim, w.dstate, generator=torch.Generator().manual_seed(5)) * 0.5
    cot = workloads.make_large_cotangents(w, batch=bsz, seqlen=L, dim=dim)
    print(f"  backward B={bsz} L={L} D={dim} bf16: {L * dim * 2 / 2**30:.2f} GiB per row", flush=True)
    chans = sample_channels(dim, k=8, seed=L + 1)
    sub = select(inp, [0], chans)
    ref = oracle.scan_bwd(*(sub.get(k) for k in TENS), dy=cot["dy"].index_select(2, torch.as_tensor(chans)),
                          dhT=cot["dhT"].index_select(1, torch.as_tensor(chans)))
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    dy, dhT = cot["dy"].to(DEV), cot["dhT"].to(DEV)
    del inp, cot
    gc.collect()
    g = ssm.scan_bwd(*(d.get(k) for k in TENS), dy=dy, dhT=dhT)
    torch.cuda.synchronize()
    ci = torch.as_tensor(chans, device=DEV)
    per_channel = {"x": 2, "delta": 2, "z": 2, "A": 0, "D": 0, "delta_bias": 0, "h0": 1}
    for k, axis in per_channel.items():
        got = g[k].index_select(axis, ci).float().cpu().double().numpy()
        check("d" + k, got, ref[k], w.dtype)
    for k in ("B", "C"):
        assert bool(torch.isfinite(g[k]).all()), f"d{k} has non-finite entries"
    del d, dy, dhT, g
    torch.cuda.empty_cache()


def test_ssd_sequence_beyond_2gib():
    w = workloads.SSD_WORKLOADS[1]
    L = 262_208
    inp = workloads.make_ssd_inputs(w, batch=1, seqlen=L, with_h0=True, seed_extra=(9,))
    print(f"  SSD B=1 L={L} H={w.nheads} P={w.headdim} N={w.dstate}: "
          f"{inp['x'].numel() * 2 / 2**30:.2f} GiB of x per row", flush=True)
    heads = [0, 37, w.nheads - 1]
    hi = torch.as_tensor(heads)
    sub = {"x": inp["x"].index_select(2, hi), "dt": inp["dt"].index_select(2, hi), "A": inp["A"][hi],
           "B": inp["B"], "C": inp["C"], "D": inp["D"][hi], "dt_bias": inp["dt_bias"][hi],
           "h0": inp["h0"].index_select(1, hi)}
    yr, hr = oracle.ssd(*(sub[k] for k in ("x", "dt", "A", "B", "C")), D=sub["D"], dt_bias=sub["dt_bias"],
                        s0=sub["h0"])
    d = {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}
    del inp
    gc.collect()
    y, hT = ssm.ssd_fwd(*(d[k] for k in ("x", "dt", "A", "B", "C", "D", "dt_bias", "h0")), return_final_state=True)
    torch.cuda.synchronize()
    hd = hi.to(DEV)
    check("y", y.index_select(2, hd).float().cpu().double().numpy(), yr, torch.bfloat16)
    check("hT", hT.index_select(1, hd).cpu().double().numpy(), hr, torch.bfloat16)
    del d, y, hT
    torch.cuda.empty_cache()
