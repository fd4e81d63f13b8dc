"""Pins of the oracle's zero-order-hold (ZOH) scan (oracle_scan_zoh_f64).

The page (youngju.dev "Mamba 논문 리뷰", section 2.2) discretises with a
zero-order hold: Abar = exp(delta A), Bbar = (delta A)^-1 (exp(delta A) - I)
delta B.  For a diagonal A the input term of state n is
(exp(delta A_n) - 1) / A_n * B_n * x, with limit delta * B_n * x at A_n = 0.
The hold is exact for an input held constant over each step, which gives the
pins their closed forms:
  - constant B and x over a run of steps of different sizes: the state is the
    exact solution of h' = A h + B x after the total time T = sum of delta,
    e^{A T} h0 + (e^{A T} - 1) / A * B x, whatever the individual steps;
  - a very long step reaches the fixed point -B x / A_n;
  - A = 0 reduces to the Euler scan (a cumulative sum of delta B x);
  - L = 1 by hand; chained calls equal one call.
Planted mistakes (the Euler term kept, the division by A_n dropped) must fail
at least one pin.
"""
import numpy as np
import pytest

import oracle


def _softplus(v):
    return np.logaddexp(0.0, v)


def pin_exact_ode_solution(orc):
    g = np.random.default_rng(1)
    Bn, L, D, N = 2, 40, 3, 5
    x = np.repeat(g.standard_normal((Bn, 1, D)), L, axis=1)
    Bm = np.repeat(g.standard_normal((Bn, 1, N)), L, axis=1)
    Cm = g.standard_normal((Bn, L, N))
    dr = g.standard_normal((Bn, L, D)) - 2.0
    A = -g.uniform(0.2, 3.0, (D, N))
    h0 = g.standard_normal((Bn, D, N))
    _, hT = orc.scan(x, dr, A, Bm, Cm, h0=h0, zoh=True)
    T = _softplus(dr).sum(axis=1)                                   # (B, D)
    eAT = np.exp(T[:, :, None] * A[None])                           # (B, D, N)
    ref = eAT * h0 + np.expm1(T[:, :, None] * A[None]) / A[None] * Bm[:, 0][:, None, :] * x[:, 0][:, :, None]
    if not np.allclose(hT, ref, rtol=1e-11, atol=1e-12):
        return f"state after T differs from the ODE solution by {np.abs(hT - ref).max():.3e}"
    return None


def pin_long_step_fixed_point(orc):
    """delta = 40 (raw step 40): exp(delta A_n) vanishes, h = -B x / A_n exactly."""
    g = np.random.default_rng(2)
    x, Bm, Cm = g.standard_normal((1, 1, 4)), g.standard_normal((1, 1, 6)), g.standard_normal((1, 1, 6))
    A = -(np.arange(6)[None, :] + 1.0) * np.ones((4, 1))
    _, hT = orc.scan(x, np.full((1, 1, 4), 40.0), A, Bm, Cm, h0=g.standard_normal((1, 4, 6)), zoh=True)
    ref = -Bm[0, 0][None, :] * x[0, 0][:, None] / A
    if not np.allclose(hT[0], ref, rtol=1e-13, atol=1e-15):
        return "long step does not reach -B x / A"
    return None


def pin_A_zero_is_euler(orc):
    g = np.random.default_rng(3)
    Bn, L, D, N = 2, 17, 3, 4
    args = (g.standard_normal((Bn, L, D)), g.standard_normal((Bn, L, D)), np.zeros((D, N)),
            g.standard_normal((Bn, L, N)), g.standard_normal((Bn, L, N)))
    kw = dict(D=g.standard_normal(D), h0=g.standard_normal((Bn, D, N)))
    y1, h1 = orc.scan(*args, **kw, zoh=True)
    y2, h2 = orc.scan(*args, **kw)
    if not np.allclose(y1, y2, rtol=1e-14, atol=1e-14) or not np.allclose(h1, h2, rtol=1e-14, atol=1e-14):
        return "A = 0 under the hold differs from the Euler scan"
    return None


def pin_L1_by_hand(orc):
    """raw step 0 (delta = ln 2), A = -1, h0 = 4, x = 2, B = C = D = 1:
    Abar = 1/2, Bbar = (1/2 - 1) / (-1) = 1/2, h1 = 2 + 1 = 3, y = 3 + 2 = 5;
    with z = ln 3 the gate is (3/4) ln 3 and y = 3.75 ln 3."""
    one = lambda v: np.full((1, 1, 1), v)
    kw = dict(D=np.ones(1), h0=np.full((1, 1, 1), 4.0), zoh=True)
    y, h = orc.scan(one(2.0), one(0.0), np.full((1, 1), -1.0), one(1.0), one(1.0), **kw)
    if abs(h.item() - 3.0) > 1e-14 or abs(y.item() - 5.0) > 1e-14:
        return f"L=1: h={h.item()} y={y.item()}, expected 3 and 5"
    y, _ = orc.scan(one(2.0), one(0.0), np.full((1, 1), -1.0), one(1.0), one(1.0), z=one(np.log(3.0)), **kw)
    if abs(y.item() - 3.75 * np.log(3.0)) > 1e-14:
        return f"L=1 with gate: y={y.item()}, expected 3.75 ln 3"
    return None


def pin_chaining(orc):
    g = np.random.default_rng(5)
    Bn, L, D, N = 2, 33, 3, 4
    x, dr = g.standard_normal((Bn, L, D)), g.standard_normal((Bn, L, D))
    A = -g.uniform(0.1, 2.0, (D, N))
    Bm, Cm, z = g.standard_normal((Bn, L, N)), g.standard_normal((Bn, L, N)), g.standard_normal((Bn, L, D))
    y, hT = orc.scan(x, dr, A, Bm, Cm, z=z, zoh=True)
    parts, h = [], None
    for a, b in [(0, 1), (1, 20), (20, 33)]:
        yy, h = orc.scan(x[:, a:b], dr[:, a:b], A, Bm[:, a:b], Cm[:, a:b], z=z[:, a:b], h0=h, zoh=True)
        parts.append(yy)
    if not np.array_equal(np.concatenate(parts, axis=1), y) or not np.array_equal(h, hT):
        return "chained calls differ from one call"
    return None


PINS = [pin_exact_ode_solution, pin_long_step_fixed_point, pin_A_zero_is_euler, pin_L1_by_hand, pin_chaining]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_zoh_pin(pin):
    msg = pin(oracle.get())
    assert msg is None, msg


@pytest.mark.parametrize("k", [26, 27])
def test_zoh_mutant_is_caught(k, tmp_path):
    orc = oracle.Oracle(oracle.build(mutant=k, out_dir=str(tmp_path)))
    assert orc.mutant == k
    failed = [p.__name__ for p in PINS if p(orc) is not None]
    assert failed, f"mutant {k} passed every zero-order-hold pin"
