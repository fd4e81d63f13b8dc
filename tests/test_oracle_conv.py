"""Pins of the oracle's conv1d + SiLU prologue (oracle_conv1d_silu_f64).

The prologue is the block's depthwise causal convolution followed by SiLU
(page youngju.dev "Mamba 논문 리뷰", section 3.4 listing: nn.Conv1d with
groups = channels, padding = d_conv - 1, output cut to the first L positions,
then F.silu).  Each pin reaches the same numbers by another route: PyTorch's
own conv1d wired as the listing wires it, scipy's causal FIR filter, numpy's
convolve over the state-extended input, scipy's expit for the SiLU, and the
chaining of calls through the carried state.  Planted mistakes (taps
reversed, one token late) must fail at least one pin.
"""
import numpy as np
import pytest
import scipy.signal
import scipy.special
import torch

import oracle


def _inputs(seed, B=2, L=37, D=5, W=4, state=False):
    g = np.random.default_rng(seed)
    x = g.standard_normal((B, L, D))
    w = g.standard_normal((D, W))
    bias = g.standard_normal(D)
    st = g.standard_normal((B, W - 1, D)) if state else None
    return x, w, bias, st


def pin_torch_conv1d(orc):
    """The section 3.4 recipe run by PyTorch: Conv1d(groups=D, padding=W-1), cut to L."""
    for W in (1, 2, 3, 4):
        x, w, bias, _ = _inputs(10 + W, W=W)
        _, pre, _ = orc.conv1d_silu(x, w, bias)
        xt = torch.from_numpy(x).transpose(1, 2)  # (B, D, L)
        ref = torch.nn.functional.conv1d(xt, torch.from_numpy(w)[:, None, :], torch.from_numpy(bias),
                                         padding=W - 1, groups=x.shape[2])[:, :, :x.shape[1]]
        ref = ref.transpose(1, 2).numpy()
        if not np.allclose(pre, ref, rtol=1e-12, atol=1e-12):
            return f"W={W}: pre differs from torch conv1d by {np.abs(pre - ref).max():.3e}"
    return None


def pin_fir_filter(orc):
    """Without a state the pre-activation is a causal FIR filter with zero initial
    conditions: scipy.signal.lfilter with numerator taps w[d, ::-1]."""
    x, w, bias, _ = _inputs(2)
    _, pre, _ = orc.conv1d_silu(x, w, bias)
    for b in range(x.shape[0]):
        for d in range(x.shape[2]):
            ref = scipy.signal.lfilter(w[d, ::-1], [1.0], x[b, :, d]) + bias[d]
            if not np.allclose(pre[b, :, d], ref, rtol=1e-12, atol=1e-12):
                return f"(b={b}, d={d}) differs from lfilter"
    return None


def pin_state_convolve(orc):
    """With a state, pre is the 'valid' convolution of [state; x] with the flipped taps."""
    x, w, bias, st = _inputs(3, state=True)
    _, pre, _ = orc.conv1d_silu(x, w, bias, st)
    for b in range(x.shape[0]):
        for d in range(x.shape[2]):
            full = np.concatenate([st[b, :, d], x[b, :, d]])
            ref = np.convolve(full, w[d, ::-1], mode="valid") + bias[d]
            if ref.shape != pre[b, :, d].shape or not np.allclose(pre[b, :, d], ref, rtol=1e-12, atol=1e-12):
                return f"(b={b}, d={d}) differs from np.convolve"
    return None


def pin_silu(orc):
    """u = pre * sigmoid(pre), with scipy's expit for the sigmoid."""
    x, w, bias, st = _inputs(4, state=True)
    u, pre, _ = orc.conv1d_silu(x * 6.0, w, bias, st)
    ref = pre * scipy.special.expit(pre)
    if not np.allclose(u, ref, rtol=1e-14, atol=1e-300):
        return f"u differs from pre*expit(pre) by {np.abs(u - ref).max():.3e}"
    return None


def pin_chaining(orc):
    """Calls chained through the carried state equal one call, bit for bit, and
    the carried state is the last W-1 input rows."""
    x, w, bias, st = _inputs(5, L=41, state=True)
    u1, _, s1 = orc.conv1d_silu(x, w, bias, st)
    if not np.array_equal(s1, x[:, -3:, :]):
        return "state_out is not the last W-1 rows of x"
    parts, s = [], st
    for a, b in [(0, 1), (1, 3), (3, 20), (20, 41)]:  # includes calls shorter than W-1
        u, _, s = orc.conv1d_silu(x[:, a:b], w, bias, s)
        parts.append(u)
    if not np.array_equal(np.concatenate(parts, axis=1), u1) or not np.array_equal(s, s1):
        return "chained calls differ from one call"
    return None


def pin_taps_by_hand(orc):
    """Single-tap kernels: w = e_k delays x by W-1-k tokens (zeros before t = 0)."""
    x, _, _, _ = _inputs(6, B=1, L=9, D=2)
    for k in range(4):
        w = np.zeros((2, 4))
        w[:, k] = 1.0
        _, pre, _ = orc.conv1d_silu(x, w)
        lag = 3 - k
        ref = np.zeros_like(x)
        ref[:, lag:, :] = x[:, :x.shape[1] - lag, :]
        if not np.array_equal(pre, ref):
            return f"tap {k}: not a delay of {lag}"
    return None


PINS = [pin_torch_conv1d, pin_fir_filter, pin_state_convolve, pin_silu, pin_chaining, pin_taps_by_hand]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_conv_pin(pin):
    msg = pin(oracle.get())
    assert msg is None, msg


def test_empty_and_short():
    orc = oracle.get()
    x = np.zeros((2, 0, 3))
    w = np.ones((3, 4))
    st = np.arange(18, dtype=np.float64).reshape(2, 3, 3)
    u, pre, s = orc.conv1d_silu(x, w, None, st)
    assert u.shape == (2, 0, 3) and np.array_equal(s, st)  # no token: the state passes through


@pytest.mark.parametrize("k", [19, 20])
def test_conv_mutant_is_caught(k, tmp_path):
    path = oracle.build(mutant=k, out_dir=str(tmp_path))
    orc = oracle.Oracle(path)
    assert orc.mutant == k
    failed = [p.__name__ for p in PINS if p(orc) is not None]
    assert failed, f"mutant {k} passed every conv pin"
