"""ssm_scan_fwd_noalloc (the forward entry point that allocates nothing: its
time-split segment summaries live in the library's own device array) against
ssm_scan_fwd given a torch-allocated workspace, through the C ABI.

Two calls in a row, the second on a smaller problem, on time-split plans
(the only plans that use scratch memory): outputs must be bitwise equal to the
workspace entry point's (same plan, same kernels), and both within the
tolerance of the fp64 oracle.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import mamba_selective_scan_06_amd as ssm
import workloads
from tests.gpu_helpers import TENSORS, check, oracle_scan, to_dev

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP GPU"),
]

# (workload, shape, time_splits): a long-context call (automatic plan, 10
# segments), then a smaller one with an explicit 3-way split, then a
# ragged fp32 one with an automatic plan.
CASES = [
    (3, dict(batch=1, seqlen=8192, dim=1536), 0),
    (1, dict(batch=1, seqlen=1000, dim=200), 3),
    (0, dict(batch=1, seqlen=700, dim=72), 0),
]


def _run(inp, d, time_splits, noalloc):
    y = torch.empty_like(d["x"])
    hT = torch.empty(d["x"].shape[0], d["x"].shape[2], d["A"].shape[1], dtype=torch.float32, device=d["x"].device)
    args = ssm.make_args(*(d.get(k) for k in TENSORS), hT=hT, y=y, time_splits=time_splits)
    plan_args = ssm.make_args(*(d.get(k) for k in TENSORS), hT=hT, y=y, time_splits=time_splits)
    nbytes = ssm.workspace_bytes(plan_args)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=d["x"].device)
    plan_args.workspace, plan_args.workspace_bytes = ws.data_ptr(), nbytes
    splits = ssm.plan(plan_args)[1]
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        rc = ssm.lib().ssm_scan_fwd_noalloc(ctypes.byref(args), ctypes.c_void_p(stream))
    else:
        rc = ssm.lib().ssm_scan_fwd(ctypes.byref(plan_args), ctypes.c_void_p(stream))
    assert rc == 0, ssm.strerror(rc)
    torch.cuda.synchronize()
    return y.float().cpu().double().numpy(), hT.cpu().double().numpy(), splits


def test_noalloc_matches_workspace_entry_point():
    for wi, shape, ts in CASES:
        w = workloads.WORKLOADS[wi]
        inp = workloads.make_inputs(w, **shape)
        d = to_dev(inp)
        print(f"case workload={w.name} shape={shape} time_splits={ts}", flush=True)
        y_ws, h_ws, splits = _run(inp, d, ts, noalloc=False)
        y_na, h_na, _ = _run(inp, d, ts, noalloc=True)
        assert splits > 1, "the case must take a time-split plan"
        assert np.array_equal(y_na, y_ws) and np.array_equal(h_na, h_ws), "no-alloc entry differs from workspace entry"
        yr, hr = oracle_scan(inp)
        check("y", y_na, yr, w.dtype)
        check("hT", h_na, hr, w.dtype)
