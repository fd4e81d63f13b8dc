"""conv1d + SiLU prologue on the GPU (ssm_conv1d_silu_fwd through the C ABI)
against the fp64 oracle on the same seeded inputs.

Tolerance: the floored max relative error of workloads.rel_err, 1e-4 for
fp32 and 2e-2 for bf16 (u is rounded once to the input dtype).  The carried
state is a copy of input rows, so it is compared bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mamba_selective_scan_06_amd as ssm
import oracle
import workloads
from tests.gpu_helpers import DEV, check, sample_channels

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP GPU"),
]

W_ = workloads.WORKLOADS


def _case(wi, batch, seqlen, dim, width=4, with_state=False, seed=0):
    w = W_[wi]
    inp = workloads.make_inputs(w, batch=batch, seqlen=seqlen, dim=dim, seed_extra=(seed,))
    prm = workloads.make_conv_params(w, dim=dim, width=width, seed_extra=(seed,))
    state = None
    if with_state:  # earlier input rows: another seeded draw of the same kind
        prev = workloads.make_inputs(w, batch=batch, seqlen=max(width - 1, 1), dim=dim, seed_extra=(seed, 1))["x"]
        state = prev[:, :width - 1].contiguous()
    return w, inp["x"], prm["weight"], prm["bias"], state


def gpu_conv(x, weight, bias, state):
    d = lambda t: None if t is None else t.to(DEV)
    u, so = ssm.conv1d_silu(d(x), d(weight), d(bias), d(state), return_state=True)
    torch.cuda.synchronize()
    return u, so


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("width", [1, 2, 3, 4])
@pytest.mark.parametrize("dim", [64, 130])  # 130: not a multiple of the 16-byte channel group
@pytest.mark.parametrize("with_state", [False, True], ids=["pad", "state"])
def test_conv_small_all_elements(dtype, width, dim, with_state):
    wi = 0 if dtype == "f32" else 1
    w, x, weight, bias, state = _case(wi, 2, 300, dim, width, with_state, seed=width)
    u, so = gpu_conv(x, weight, bias, state)
    ur, _, sr = oracle.conv1d_silu(x, weight, bias, state)
    check("u", u.float().cpu().double().numpy(), ur, w.dtype)
    exp_state = x[:, x.shape[1] - (width - 1):, :]
    assert torch.equal(so.cpu(), exp_state), "state_out is not the last W-1 input rows"


@pytest.mark.parametrize("L", [1, 2, 3, 5, 64, 65, 131])
def test_conv_lengths_and_no_bias(L):
    """Runs shorter than W-1, exactly one 64-token run, one past it, a ragged tail."""
    w, x, weight, _, state = _case(1, 3, L, 96, 4, True, seed=L)
    u, so = gpu_conv(x, weight, None, state)
    ur, _, sr = oracle.conv1d_silu(x, weight, None, state)
    check("u", u.float().cpu().double().numpy(), ur, w.dtype)
    ref_state = torch.cat([state, x], dim=1)[:, -3:, :]
    assert torch.equal(so.cpu(), ref_state)


def test_conv_chained_calls_equal_one_call():
    """A long sequence fed in calls of uneven length through the carried state
    gives the single call's output bit for bit (same inputs to every product)."""
    w, x, weight, bias, _ = _case(1, 2, 1000, 256, 4, False, seed=9)
    dx, dw, db = x.to(DEV), weight.to(DEV), bias.to(DEV)
    u1, s1 = ssm.conv1d_silu(dx, dw, db, return_state=True)
    parts, st = [], None
    for a, b in [(0, 2), (2, 3), (3, 400), (400, 1000)]:
        u, st = ssm.conv1d_silu(dx[:, a:b].contiguous(), dw, db, st, return_state=True)
        parts.append(u)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts, dim=1), u1) and torch.equal(st, s1)
    ur, _, _ = oracle.conv1d_silu(x, weight, bias)
    check("u", u1.float().cpu().double().numpy(), ur, w.dtype)


def test_conv_empty_sequence_passes_state():
    x = torch.empty(2, 0, 64, dtype=torch.bfloat16, device=DEV)
    weight = torch.randn(64, 4, device=DEV)
    state = torch.randn(2, 3, 64, device=DEV).to(torch.bfloat16)
    u, so = ssm.conv1d_silu(x, weight, None, state, return_state=True)
    torch.cuda.synchronize()
    assert u.shape == (2, 0, 64) and torch.equal(so, state)
    _, so = ssm.conv1d_silu(x, weight, return_state=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(so) == 0


def test_conv_w2_full_size_sampled():
    """The 1.4B-shaped layer's x (B4 L8192 D4096 bf16), launched as the bench
    launches it; sampled channels against the oracle (channels are independent)."""
    w = W_[2]
    x = workloads.make_inputs(w)["x"]
    prm = workloads.make_conv_params(w)
    u, so = gpu_conv(x, prm["weight"], prm["bias"], None)
    didx = sample_channels(w.dim, k=32, seed=5)
    di = torch.tensor(didx)
    ur, _, _ = oracle.conv1d_silu(x.index_select(2, di), prm["weight"].index_select(0, di),
                                  prm["bias"].index_select(0, di))
    check("u", u.index_select(2, di.to(DEV)).float().cpu().double().numpy(), ur, w.dtype)
    assert torch.equal(so.cpu(), x[:, -3:, :])
