"""Pins of the oracle's Mamba-2 state-space dual layer (oracle_ssd_f64).

The page (youngju.dev "Mamba 논문 리뷰", section 4.1) states the duality: the
recurrence h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t is the same map as a
structured masked attention Y = (T o M) X, T the causal mask.  The oracle runs
the recurrence; the pins reach the same numbers by:
  - the dual quadratic form, built with numpy matrix products;
  - the Mamba-1 selective-scan oracle run on the head's channels (a head is
    Mamba-1 with its step size shared by its P channels and one decay rate
    A[h] for every state), which the forward pins tie to closed forms;
  - chained calls through the carried state;
  - A = 0, where the state is a plain cumulative sum.
Planted mistakes (step size left out of the decay, B read out in place of C)
must fail at least one pin.
"""
import numpy as np
import pytest

import oracle


def _inputs(seed, B=2, L=23, H=4, P=3, G=2, N=5, state=True):
    g = np.random.default_rng(seed)
    return dict(
        x=g.standard_normal((B, L, H, P)), dt=g.standard_normal((B, L, H)), A=-g.uniform(0.1, 2.0, H),
        B=g.standard_normal((B, L, G, N)), C=g.standard_normal((B, L, G, N)), D=g.standard_normal(H),
        dt_bias=g.standard_normal(H), s0=g.standard_normal((B, H, P, N)) if state else None)


def _softplus(v):
    return np.logaddexp(0.0, v)


def pin_dual_form(orc):
    """y = (causal mask o M) X + decayed initial-state readout + D x, with
    M[t, s] = (C_t . B_s) exp(sum_{s<r<=t} delta_r A) delta_s."""
    I = _inputs(1)
    y, _ = orc.ssd(**I)
    Bn, L, H, P = I["x"].shape
    G = I["B"].shape[2]
    for b in range(Bn):
        for h in range(H):
            g = h // (H // G)
            delta = _softplus(I["dt"][b, :, h] + I["dt_bias"][h])
            cs = np.cumsum(delta * I["A"][h])                       # log of the decay from 0 to t
            CB = I["C"][b, :, g, :] @ I["B"][b, :, g, :].T          # (L, L): C_t . B_s
            decay = np.exp(cs[:, None] - cs[None, :])
            M = np.tril(CB * decay * delta[None, :])
            Y = M @ I["x"][b, :, h, :]                              # (L, P)
            Y += np.exp(cs)[:, None] * (I["C"][b, :, g, :] @ I["s0"][b, h].T)
            Y += I["D"][h] * I["x"][b, :, h, :]
            if not np.allclose(y[b, :, h, :], Y, rtol=1e-10, atol=1e-10):
                return f"(b={b}, h={h}) differs from the dual form by {np.abs(y[b, :, h, :] - Y).max():.3e}"
    return None


def pin_mamba1_heads(orc):
    """Each group's heads equal the selective scan over channels (h, p) with the
    head's step size and a constant decay rate A[h] across states."""
    I = _inputs(2)
    y, sT = orc.ssd(**I)
    Bn, L, H, P = I["x"].shape
    G, N = I["B"].shape[2], I["B"].shape[3]
    hpg = H // G
    for g in range(G):
        hs = slice(g * hpg, (g + 1) * hpg)
        x1 = I["x"][:, :, hs, :].reshape(Bn, L, hpg * P)
        dt1 = np.repeat(I["dt"][:, :, hs], P, axis=2)
        A1 = np.repeat(I["A"][hs], P)[:, None] * np.ones((1, N))
        D1 = np.repeat(I["D"][hs], P)
        b1 = np.repeat(I["dt_bias"][hs], P)
        h01 = I["s0"][:, hs].reshape(Bn, hpg * P, N)
        y1, hT1 = orc.scan(x1, dt1, A1, I["B"][:, :, g, :], I["C"][:, :, g, :], D1, None, b1, h01)
        if not np.allclose(y[:, :, hs, :].reshape(Bn, L, hpg * P), y1, rtol=1e-12, atol=1e-12):
            return f"group {g}: y differs from the selective scan"
        if not np.allclose(sT[:, hs].reshape(Bn, hpg * P, N), hT1, rtol=1e-12, atol=1e-12):
            return f"group {g}: final state differs from the selective scan"
    return None


def pin_chaining(orc):
    I = _inputs(3, L=30)
    y, sT = orc.ssd(**I)
    parts, s = [], I["s0"]
    for a, b in [(0, 1), (1, 11), (11, 30)]:
        J = dict(I, x=I["x"][:, a:b], dt=I["dt"][:, a:b], B=I["B"][:, a:b], C=I["C"][:, a:b], s0=s)
        yy, s = orc.ssd(**J)
        parts.append(yy)
    if not np.array_equal(np.concatenate(parts, axis=1), y) or not np.array_equal(s, sT):
        return "chained calls differ from one call"
    return None


def pin_A_zero(orc):
    """A = 0: no decay, S_t = S_0 + sum_{s<=t} delta_s x_s B_s^T."""
    I = _inputs(4, G=1)
    I["A"] = np.zeros_like(I["A"])
    y, sT = orc.ssd(**I)
    delta = _softplus(I["dt"] + I["dt_bias"][None, None, :])          # (B, L, H)
    inc = np.einsum("blh,blhp,bln->blhpn", delta, I["x"], I["B"][:, :, 0, :])
    S = I["s0"][:, None] + np.cumsum(inc, axis=1)                      # (B, L, H, P, N)
    Y = np.einsum("bln,blhpn->blhp", I["C"][:, :, 0, :], S) + I["D"][None, None, :, None] * I["x"]
    if not np.allclose(y, Y, rtol=1e-11, atol=1e-11) or not np.allclose(sT, S[:, -1], rtol=1e-11, atol=1e-11):
        return "A = 0 differs from the cumulative sum"
    return None


PINS = [pin_dual_form, pin_mamba1_heads, pin_chaining, pin_A_zero]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_ssd_pin(pin):
    msg = pin(oracle.get())
    assert msg is None, msg


@pytest.mark.parametrize("k", [21, 22])
def test_ssd_mutant_is_caught(k, tmp_path):
    orc = oracle.Oracle(oracle.build(mutant=k, out_dir=str(tmp_path)))
    assert orc.mutant == k
    failed = [p.__name__ for p in PINS if p(orc) is not None]
    assert failed, f"mutant {k} passed every SSD pin"
