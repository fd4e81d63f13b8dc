"""Pins of the oracle's backward pass (CPU only).

The gradients of oracle_scan_bwd_f64 are checked against central finite
differences of the forward oracle, an independent computation, on every
element of every input, for the scalar loss sum(dy * y) + sum(dhT * hT).
Shapes are tiny so that the few thousand forward calls stay fast.  Each
backward mutant planted behind ORACLE_MUTANT (decay missing from the carried
adjoint, sign of the decay term, dL/dhT dropped, softplus derivative
missing) must fail this pin.  The zero-order-hold gradients (youngju.dev
section 2.2's input term (exp(delta A) - 1) / A B x) are pinned the same way
against the zero-order-hold forward, including steps where delta A is tiny
(the series branch of dc/dA) or A is exactly 0; the mutants that leave the
hold's own dependence on A out of dA, or keep the Euler term's derivative in
delta, must fail.
"""
import numpy as np
import pytest

import oracle

EPS = 1e-6
TOL = 1e-6  # finite differences in fp64 at EPS reach ~1e-9 here


def _problem(seed, B=2, L=5, D=3, N=4, gate=True, skip=True, bias=True, h0=True, dhT=True):
    g = np.random.default_rng(seed)
    p = {
        "x": g.normal(size=(B, L, D)), "delta": g.normal(size=(B, L, D)),
        "A": -np.exp(g.normal(size=(D, N))), "B": g.normal(size=(B, L, N)), "C": g.normal(size=(B, L, N)),
        "D": g.normal(size=D) if skip else None, "z": g.normal(size=(B, L, D)) if gate else None,
        "delta_bias": 0.5 * g.normal(size=D) if bias else None,
        "h0": g.normal(size=(B, D, N)) if h0 else None,
    }
    cot = {"dy": g.normal(size=(B, L, D)), "dhT": g.normal(size=(B, D, N)) if dhT else None}
    return p, cot


def _loss(orc, p, cot, zoh=False):
    y, hT = orc.scan(**p, threads=1, zoh=zoh)
    val = float((cot["dy"] * y).sum())
    if cot["dhT"] is not None:
        val += float((cot["dhT"] * hT).sum())
    return val


def fd_errors(orc, p, cot, zoh=False):
    """max |fd - analytic| / max |fd| per input (h0 included even when absent)."""
    grads = orc.scan_bwd(**p, dy=cot["dy"], dhT=cot["dhT"], zoh=zoh)
    errs = {}
    for name, arr in p.items():
        if arr is None and name != "h0":
            assert name not in grads
            continue
        base = arr if arr is not None else np.zeros_like(grads["h0"])
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] += EPS
            minus[idx] -= EPS
            fd[idx] = (_loss(orc, {**p, name: plus}, cot, zoh) - _loss(orc, {**p, name: minus}, cot, zoh)) / (2 * EPS)
        scale = max(float(np.abs(fd).max()), 1e-12)
        errs[name] = float(np.abs(fd - grads[name]).max()) / scale
    return errs


CASES = {
    "full": {},
    "no-gate-no-skip": dict(gate=False, skip=False),
    "no-bias-no-h0": dict(bias=False, h0=False),
    "no-dhT": dict(dhT=False),
    "L1": dict(L=1),
    "N1": dict(N=1, D=2),
}


@pytest.mark.parametrize("case", list(CASES))
def test_gradients_match_finite_differences(case):
    p, cot = _problem(11, **CASES[case])
    errs = fd_errors(oracle.get(), p, cot)
    assert max(errs.values()) < TOL, errs


def test_zero_cotangent_gives_zero_gradients():
    p, cot = _problem(3)
    g = oracle.scan_bwd(**p, dy=np.zeros_like(cot["dy"]), dhT=None)
    assert all(np.all(v == 0.0) for v in g.values())


def test_gradients_are_linear_in_the_cotangents():
    p, cot = _problem(5)
    g1 = oracle.scan_bwd(**p, dy=cot["dy"], dhT=cot["dhT"])
    g2 = oracle.scan_bwd(**p, dy=2.5 * cot["dy"], dhT=2.5 * cot["dhT"])
    for k in g1:
        np.testing.assert_allclose(g2[k], 2.5 * g1[k], rtol=1e-12, atol=1e-14)


BWD_MUTANTS = [15, 16, 17, 18]


@pytest.mark.parametrize("k", BWD_MUTANTS)
def test_backward_mutant_is_caught(k, tmp_path):
    orc = oracle.Oracle(oracle.build(mutant=k, out_dir=str(tmp_path)))
    assert orc.mutant == k
    p, cot = _problem(11)
    errs = fd_errors(orc, p, cot)
    assert max(errs.values()) > 1e-3, f"backward mutant {k} passed the finite-difference pin: {errs}"


ZOH_CASES = {
    "full": {},
    "no-gate-no-skip-no-h0": dict(gate=False, skip=False, h0=False),
    "no-dhT-L1": dict(dhT=False, L=1),
}


@pytest.mark.parametrize("case", list(ZOH_CASES))
def test_zoh_gradients_match_finite_differences(case):
    p, cot = _problem(12, **ZOH_CASES[case])
    errs = fd_errors(oracle.get(), p, cot, zoh=True)
    assert max(errs.values()) < TOL, errs


def test_zoh_gradients_small_and_zero_decay_rates():
    """A_n of 1e-5 (|delta A_n| < 1e-3: the series branch of dc/dA) and A_n = 0
    (the coefficient's limit delta, derivative delta^2 / 2), beside ordinary
    rates."""
    p, cot = _problem(13, D=3, N=4)
    p["A"][0, :] = -1e-5 * np.exp(np.random.default_rng(1).normal(size=4))
    p["A"][1, 1] = 0.0
    p["A"][2, 3] = 0.0
    errs = fd_errors(oracle.get(), p, cot, zoh=True)
    assert max(errs.values()) < TOL, errs


def test_zoh_gradients_differ_from_euler():
    """The hold changes every gradient that the input term reaches (a pin that
    the zoh switch is not ignored), and not dL/dh0: the adjoint carried back to
    the initial state is the decays' product applied to the cotangents, and
    dL/dD sums dy SiLU(z) x; the input term enters neither."""
    p, cot = _problem(14)
    ge = oracle.scan_bwd(**p, dy=cot["dy"], dhT=cot["dhT"])
    gz = oracle.scan_bwd(**p, dy=cot["dy"], dhT=cot["dhT"], zoh=True)
    for k in ("x", "delta", "A", "B", "C", "z"):
        assert np.abs(ge[k] - gz[k]).max() > 1e-3 * np.abs(ge[k]).max(), k
    np.testing.assert_array_equal(ge["h0"], gz["h0"])
    np.testing.assert_array_equal(ge["D"], gz["D"])


@pytest.mark.parametrize("k", [28, 29])
def test_zoh_backward_mutant_is_caught(k, tmp_path):
    orc = oracle.Oracle(oracle.build(mutant=k, out_dir=str(tmp_path)))
    assert orc.mutant == k
    p, cot = _problem(12)
    errs = fd_errors(orc, p, cot, zoh=True)
    assert max(errs.values()) > 1e-3, f"backward mutant {k} passed the finite-difference pin: {errs}"
