"""Pins of the oracle's gated-linear-attention / mLSTM recurrence (oracle_gla_f64).

The HedgeMamba review (stage 2) writes linear attention as the recurrence
s_t = s_{t-1} + phi(k_t)^T v_t, the causal form of phi(Q) (phi(K)^T V), with
elu + 1 as the example feature map; the xLSTM review's mLSTM scales the
previous matrix state by a forget coefficient and adds the input-gated outer
product of value and key.  The oracle runs that recurrence; the pins reach the
same numbers by:
  - the causal quadratic form tril(Q K^T) V built with numpy matrix products,
    with and without gates (decay exp(sum of log f) between key and query);
  - the feature map applied beforehand with torch's elu;
  - the SSD oracle (pinned on its own) with log f = delta A and i = delta;
  - chained calls through the carried state;
  - one step worked by hand.
Planted mistakes (readout before the update, feature map left off q, input
gate applied to the carried state) must fail at least one pin.
"""
import numpy as np
import pytest
import torch

import oracle


def _inputs(seed, B=2, L=21, H=4, P=3, G=2, N=5, gates=True, state=True):
    g = np.random.default_rng(seed)
    return dict(
        q=g.standard_normal((B, L, G, N)), k=g.standard_normal((B, L, G, N)), v=g.standard_normal((B, L, H, P)),
        log_f=-g.uniform(0.01, 1.0, (B, L, H)) if gates else None,
        in_gate=g.uniform(0.1, 2.0, (B, L, H)) if gates else None,
        s0=g.standard_normal((B, H, P, N)) if state else None)


def _quadratic(I, fm=False):
    """Causal attention form: y_t = sum_{s<=t} D[t,s] i_s (q_t . k_s) v_s + exp(cs_t) q_t S0^T,
    D[t,s] = exp(cs_t - cs_s), cs the running sum of log f."""
    phi = (lambda u: torch.nn.functional.elu(torch.from_numpy(u)).numpy() + 1.0) if fm else (lambda u: u)
    Bn, L, H, P = I["v"].shape
    G = I["k"].shape[2]
    Y = np.zeros_like(I["v"])
    for b in range(Bn):
        for h in range(H):
            g = h // (H // G)
            Q, K, V = phi(I["q"][b, :, g]), phi(I["k"][b, :, g]), I["v"][b, :, h]
            lf = I["log_f"][b, :, h] if I["log_f"] is not None else np.zeros(L)
            ig = I["in_gate"][b, :, h] if I["in_gate"] is not None else np.ones(L)
            cs = np.cumsum(lf)
            W = np.tril((Q @ K.T) * np.exp(cs[:, None] - cs[None, :]) * ig[None, :])
            Y[b, :, h] = W @ V
            if I["s0"] is not None:
                Y[b, :, h] += np.exp(cs)[:, None] * (Q @ I["s0"][b, h].T)
    return Y


def pin_linear_attention(orc):
    """No gates, no feature map, no state: y = tril(Q K^T) V."""
    I = _inputs(1, gates=False, state=False)
    y, _ = orc.gla(**I)
    Y = _quadratic(I)
    if not np.allclose(y, Y, rtol=1e-11, atol=1e-11):
        return f"linear attention differs from tril(QK^T)V by {np.abs(y - Y).max():.3e}"
    return None


def pin_gated_quadratic(orc):
    I = _inputs(2)
    y, _ = orc.gla(**I)
    Y = _quadratic(I)
    if not np.allclose(y, Y, rtol=1e-11, atol=1e-11):
        return f"gated recurrence differs from the gated quadratic form by {np.abs(y - Y).max():.3e}"
    return None


def pin_feature_map(orc):
    """feature_map = elu + 1 on q and k equals feeding torch's elu(q) + 1 and elu(k) + 1."""
    I = _inputs(3)
    y1, s1 = orc.gla(**I, feature_map=True)
    J = dict(I)
    for n in ("q", "k"):
        J[n] = torch.nn.functional.elu(torch.from_numpy(I[n])).numpy() + 1.0
    y2, s2 = orc.gla(**J, feature_map=False)
    if not np.allclose(y1, y2, rtol=1e-13, atol=1e-13) or not np.allclose(s1, s2, rtol=1e-13, atol=1e-13):
        return "feature map differs from elu + 1 applied beforehand"
    if not np.allclose(y1, _quadratic(I, fm=True), rtol=1e-11, atol=1e-11):
        return "feature map differs from the quadratic form"
    return None


def pin_ssd_special_case(orc):
    """log f = delta A[h] and i = delta with delta = softplus(dt + dt_bias) is the SSD layer without D."""
    g = np.random.default_rng(4)
    B, L, H, P, G, N = 2, 19, 4, 3, 2, 5
    x, dt = g.standard_normal((B, L, H, P)), g.standard_normal((B, L, H))
    A, bias = -g.uniform(0.1, 2.0, H), g.standard_normal(H)
    Bm, Cm, s0 = g.standard_normal((B, L, G, N)), g.standard_normal((B, L, G, N)), g.standard_normal((B, H, P, N))
    y1, s1 = orc.ssd(x, dt, A, Bm, Cm, None, bias, s0)
    delta = np.logaddexp(0.0, dt + bias[None, None, :])
    y2, s2 = orc.gla(Cm, Bm, x, log_f=delta * A[None, None, :], in_gate=delta, s0=s0)
    if not np.allclose(y1, y2, rtol=1e-12, atol=1e-12) or not np.allclose(s1, s2, rtol=1e-12, atol=1e-12):
        return "gated form with SSD gates differs from the SSD oracle"
    return None


def pin_chaining(orc):
    I = _inputs(5, L=30)
    y, sT = orc.gla(**I, feature_map=True)
    parts, s = [], I["s0"]
    for a, b in [(0, 1), (1, 12), (12, 30)]:
        J = dict(I, q=I["q"][:, a:b], k=I["k"][:, a:b], v=I["v"][:, a:b], log_f=I["log_f"][:, a:b],
                 in_gate=I["in_gate"][:, a:b], s0=s)
        yy, s = orc.gla(**J, feature_map=True)
        parts.append(yy)
    if not np.array_equal(np.concatenate(parts, axis=1), y) or not np.array_equal(s, sT):
        return "chained calls differ from one call"
    return None


def pin_one_step_by_hand(orc):
    """P = N = 1, f = 1/2, i = 3, v = 2, k = 1.5, q = -1, S0 = 4: S1 = 2 + 9 = 11, y = -11;
    with elu + 1: phi(k) = 2.5, phi(q) = 1/e: S1 = 2 + 15 = 17, y = 17/e."""
    one = lambda val, shape: np.full(shape, val)
    args = dict(q=one(-1.0, (1, 1, 1, 1)), k=one(1.5, (1, 1, 1, 1)), v=one(2.0, (1, 1, 1, 1)),
                log_f=one(-np.log(2.0), (1, 1, 1)), in_gate=one(3.0, (1, 1, 1)), s0=one(4.0, (1, 1, 1, 1)))
    y, s = orc.gla(**args)
    if abs(s.item() - 11.0) > 1e-14 or abs(y.item() + 11.0) > 1e-14:
        return f"one step: S1={s.item()} y={y.item()}, expected 11 and -11"
    y, s = orc.gla(**args, feature_map=True)
    if abs(s.item() - 17.0) > 1e-14 or abs(y.item() - 17.0 / np.e) > 1e-14:
        return f"one step with elu+1: S1={s.item()} y={y.item()}, expected 17 and 17/e"
    return None


PINS = [pin_linear_attention, pin_gated_quadratic, pin_feature_map, pin_ssd_special_case, pin_chaining,
        pin_one_step_by_hand]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_gla_pin(pin):
    msg = pin(oracle.get())
    assert msg is None, msg


def test_empty_sequence_passes_state():
    I = _inputs(6, L=0)
    y, s = oracle.get().gla(**I)
    assert y.shape == (2, 0, 4, 3) and np.array_equal(s, I["s0"])


@pytest.mark.parametrize("k", [23, 24, 25])
def test_gla_mutant_is_caught(k, tmp_path):
    orc = oracle.Oracle(oracle.build(mutant=k, out_dir=str(tmp_path)))
    assert orc.mutant == k
    failed = [p.__name__ for p in PINS if p(orc) is not None]
    assert failed, f"mutant {k} passed every gated-linear-attention pin"
