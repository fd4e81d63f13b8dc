"""Closed-form pins for the fp64 oracle.

Each check takes an oracle handle and raises AssertionError when the oracle
disagrees with something fixed independently of it: values derived by hand
(tests/golden), closed forms of special cases, a library routine standing in
for one step, a brute-force unrolled sum, or an invariant of the recurrence.
They are collected by test_oracle.py and replayed against deliberately broken
builds of the oracle by test_oracle_mutants.py.

Passages (page youngju.dev "Mamba 논문 리뷰"): section 2.2 discretisation and
recurrence, section 3.1 softplus selection, section 3.3 selective_scan listing
(tensor contract, Euler input term, update-then-read), section 3.4 skip D and
SiLU(z) gate.  Linear attention as the A = 0 relative: page suanlab.com,
"2단계" (s_t = s_{t-1} + phi(k_t)^T v_t).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _softplus_lib(v):
    # numpy's logaddexp(0, v) = log(e^0 + e^v): an independent library routine
    return np.logaddexp(0.0, v)


def _silu(z):
    return z * (0.5 * (1.0 + np.tanh(0.5 * z)))  # z * sigmoid(z) via tanh


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    assert np.all(err <= lim), f"{what}: max err {err.max():.3e} (rtol {rtol}, atol {atol})"


def _rand_case(seed, bsz=2, L=37, dim=5, N=4, gate=True, skip=True, bias=True, h0=True):
    g = _rng(seed)
    c = {
        "x": g.standard_normal((bsz, L, dim)),
        "delta": g.standard_normal((bsz, L, dim)),
        "A": -g.uniform(0.2, 3.0, size=(dim, N)),
        "B": g.standard_normal((bsz, L, N)),
        "C": g.standard_normal((bsz, L, N)),
        "D": g.standard_normal(dim) if skip else None,
        "z": g.standard_normal((bsz, L, dim)) if gate else None,
        "delta_bias": g.uniform(-3.0, 0.5, size=dim) if bias else None,
        "h0": g.standard_normal((bsz, dim, N)) if h0 else None,
    }
    return c


# ---------------------------------------------------------------- softplus --
def check_softplus_values(orc):
    """softplus(0) = ln 2; softplus(v) - softplus(-v) = v; large |v| limits;
    agreement with numpy's logaddexp over a grid."""
    v = np.array([0.0])
    _close(orc.softplus(v), [math.log(2.0)], 1e-15, what="softplus(0)")
    grid = np.linspace(-60.0, 60.0, 2401)
    sp = orc.softplus(grid)
    _close(sp, _softplus_lib(grid), 1e-13, what="softplus vs logaddexp")
    _close(sp - orc.softplus(-grid), grid, 1e-13, 1e-13, what="softplus(v)-softplus(-v)=v")
    big = np.array([800.0, -800.0, 40.0, -40.0])
    _close(orc.softplus(big), [800.0, 0.0, 40.0 + math.exp(-40.0), math.exp(-40.0)], 1e-15,
           what="softplus large |v|")


# ------------------------------------------------------------ hand values --
def check_l1_by_hand(orc):
    with open(os.path.join(GOLDEN, "l1_by_hand.json")) as f:
        gld = json.load(f)
    i, e = gld["inputs"], gld["expected"]
    one = lambda v: np.full((1, 1, 1), v)
    args = dict(x=one(i["x"]), delta=one(i["delta"]), A=np.full((1, 1), i["A"]),
                B=one(i["B"]), C=one(i["C"]), D=np.full(1, i["D"]), h0=one(i["h0"]))
    y, hT = orc.scan(**args)
    _close(hT.ravel(), [e["hT"]], 1e-14, what="L=1 hT")
    _close(y.ravel(), [e["y_no_gate"]], 1e-14, what="L=1 y")
    y, _ = orc.scan(**args, z=one(i["z"]))
    _close(y.ravel(), [e["y_gated"]], 1e-14, what="L=1 gated y")


def check_l2_n2_by_hand(orc):
    with open(os.path.join(GOLDEN, "l2_n2_by_hand.json")) as f:
        gld = json.load(f)
    i, e = gld["inputs"], gld["expected"]
    x = np.array(i["x"]).reshape(1, 2, 1)
    delta = np.array(i["delta"]).reshape(1, 2, 1)
    A = np.array(i["A"]).reshape(1, 2)
    B = np.array(i["B"]).reshape(1, 2, 2)
    C = np.array(i["C"]).reshape(1, 2, 2)
    y, hT = orc.scan(x, delta, A, B, C, D=np.full(1, i["D"]))
    _close(y.ravel(), e["y"], 1e-14, what="L=2 N=2 y")
    _close(hT.ravel(), e["hT"], 1e-14, what="L=2 N=2 hT")


# ----------------------------------------------------------- closed forms --
def check_A_zero_is_cumsum(orc):
    """A = 0 makes Abar = I: the state is h0 plus a running sum of delta*B*x
    (the linear-attention form s_t = s_{t-1} + k_t^T v_t)."""
    c = _rand_case(11, bsz=2, L=50, dim=3, N=4)
    c["A"] = np.zeros_like(c["A"])
    y, hT = orc.scan(**c)
    dt = _softplus_lib(c["delta"] + c["delta_bias"][None, None, :])          # (B,L,D)
    inc = dt[..., None] * c["B"][:, :, None, :] * c["x"][..., None]           # (B,L,D,N)
    h = c["h0"][:, None, :, :] + np.cumsum(inc, axis=1)                      # (B,L,D,N)
    yr = np.einsum("bln,bldn->bld", c["C"], h) + c["D"][None, None, :] * c["x"]
    yr = yr * _silu(c["z"])
    _close(y, yr, 1e-11, 1e-12, what="A=0 y")
    _close(hT, h[:, -1], 1e-11, 1e-12, what="A=0 hT")


def check_constant_inputs_geometric(orc):
    """Constant delta, B, x give h_t = a^t h0 + b (1 - a^t) / (1 - a)."""
    L, N = 100, 5
    A = -np.array([[0.1, 0.5, 1.0, 2.0, 7.0]])
    raw, Bv, xv, h0v = -1.3, np.array([0.7, -1.1, 2.0, 0.4, -0.9]), 1.7, np.array([0.5, -2.0, 1.0, 3.0, 0.25])
    x = np.full((1, L, 1), xv)
    delta = np.full((1, L, 1), raw)
    B = np.tile(Bv, (1, L, 1))
    C = np.zeros((1, L, N)); C[:, :, 2] = 1.0   # read out state n = 2 only
    y, hT = orc.scan(x, delta, A, B, C, h0=h0v.reshape(1, 1, N))
    dt = float(_softplus_lib(raw))
    a = np.exp(dt * A[0])
    b = dt * Bv * xv
    t = np.arange(1, L + 1)[:, None]
    h = a ** t * h0v + b * (1.0 - a ** t) / (1.0 - a)
    _close(hT[0, 0], h[-1], 1e-12, what="geometric hT")
    _close(y[0, :, 0], h[:, 2], 1e-12, what="geometric y")


def check_bruteforce_unrolled(orc):
    """h_t = exp(A sum_{r<=t} dt_r) h0 + sum_{s<=t} exp(A sum_{s<r<=t} dt_r) dt_s B_s x_s,
    evaluated directly for every t (O(L^2)), with products of Abar written as
    exponentials of sums."""
    c = _rand_case(23, bsz=2, L=19, dim=3, N=3)
    y, hT = orc.scan(**c)
    bsz, L, dim = c["x"].shape
    N = c["A"].shape[1]
    dt = _softplus_lib(c["delta"] + c["delta_bias"][None, None, :])
    yr = np.zeros_like(y)
    hl = np.zeros((bsz, dim, N))
    for b in range(bsz):
        for d in range(dim):
            for t in range(L):
                h = np.exp(c["A"][d] * dt[b, : t + 1, d].sum()) * c["h0"][b, d]
                for s in range(t + 1):
                    h = h + np.exp(c["A"][d] * dt[b, s + 1: t + 1, d].sum()) * dt[b, s, d] * c["B"][b, s] * c["x"][b, s, d]
                yr[b, t, d] = (c["C"][b, t] @ h + c["D"][d] * c["x"][b, t, d]) * _silu(c["z"][b, t, d])
                if t == L - 1:
                    hl[b, d] = h
    _close(y, yr, 1e-11, 1e-13, what="brute-force y")
    _close(hT, hl, 1e-11, 1e-13, what="brute-force hT")


def check_assoc_twin(orc):
    """The log-depth associative scan over (a, b) pairs equals the sequential loop."""
    for seed, L in ((31, 1), (32, 64), (33, 257)):
        c = _rand_case(seed, bsz=2, L=L, dim=3, N=4)
        y1, h1 = orc.scan(**c)
        y2, h2 = orc.assoc_scan(**c)
        _close(y2, y1, 1e-12, 1e-13, what=f"assoc y L={L}")
        _close(h2, h1, 1e-12, 1e-13, what=f"assoc hT L={L}")


# ------------------------------------------------------------- invariants --
def check_chunked_equals_full(orc):
    """Passing hT of one call as h0 of the next gives bitwise the one-call result."""
    c = _rand_case(41, bsz=2, L=90, dim=4, N=4)
    y, hT = orc.scan(**c)
    h = c["h0"]
    parts = []
    for lo, hi in ((0, 1), (1, 33), (33, 64), (64, 90)):
        sl = {k: (v[:, lo:hi] if k in ("x", "delta", "B", "C", "z") else v) for k, v in c.items()}
        sl["h0"] = h
        yp, h = orc.scan(**sl)
        parts.append(yp)
    assert np.array_equal(np.concatenate(parts, axis=1), y), "chunked y differs"
    assert np.array_equal(h, hT), "chunked hT differs"


def check_causality(orc):
    """Changing the inputs at t0 leaves y_t for t < t0 unchanged and changes y_t0."""
    c = _rand_case(51, bsz=1, L=40, dim=3, N=4)
    y, _ = orc.scan(**c)
    t0 = 17
    for key in ("x", "delta", "B", "C", "z"):
        c2 = {k: (None if v is None else v.copy()) for k, v in c.items()}
        c2[key][:, t0] += 0.75
        y2, _ = orc.scan(**c2)
        assert np.array_equal(y2[:, :t0], y[:, :t0]), f"perturbing {key} changed the past"
        assert not np.array_equal(y2[:, t0], y[:, t0]), f"perturbing {key} did not change y[t0]"


def check_linearity(orc):
    """Without the gate, y and hT are linear in (x, h0) jointly."""
    c = _rand_case(61, bsz=2, L=30, dim=3, N=4, gate=False)
    g = _rng(62)
    x2, h2 = g.standard_normal(c["x"].shape), g.standard_normal(c["h0"].shape)
    al, be = 0.7, -1.9
    ya, ha = orc.scan(**c)
    cb = dict(c, x=x2, h0=h2)
    yb, hb = orc.scan(**cb)
    cc = dict(c, x=al * c["x"] + be * x2, h0=al * c["h0"] + be * h2)
    yc, hc = orc.scan(**cc)
    _close(yc, al * ya + be * yb, 1e-11, 1e-12, what="linearity y")
    _close(hc, al * ha + be * hb, 1e-11, 1e-12, what="linearity hT")


def check_gate_and_readout_special_cases(orc):
    """z = 0 gives y = 0; C = 0 gives y = D x SiLU(z); no skip and no gate with
    C = e_n reads out state n."""
    c = _rand_case(71, bsz=1, L=25, dim=3, N=4)
    cz = dict(c, z=np.zeros_like(c["z"]))
    y, _ = orc.scan(**cz)
    assert np.all(y == 0.0), "z = 0 must zero the output"
    cc = dict(c, C=np.zeros_like(c["C"]))
    y, _ = orc.scan(**cc)
    _close(y, c["D"][None, None, :] * c["x"] * _silu(c["z"]), 1e-13, 1e-15, what="C = 0")
    # reading out one state at every step reproduces that state's trajectory
    e = np.zeros_like(c["C"]); e[:, :, 3] = 1.0
    y, hT = orc.scan(**dict(c, C=e, z=None, D=None))
    _close(y[:, -1, :], hT[:, :, 3], 1e-15, what="C = e_3 readout")


def check_delta_limits(orc):
    """delta -> 0 keeps the state (Abar -> 1, no input); a large delta with A <= -1
    forgets it (Abar -> 0), leaving h_t = delta B_t x_t."""
    c = _rand_case(81, bsz=1, L=12, dim=2, N=3, gate=False, skip=False, bias=False)
    c["A"] = -np.abs(c["A"]) - 1.0
    keep = dict(c, delta=np.full_like(c["delta"], -80.0))
    _, hT = orc.scan(**keep)
    _close(hT, c["h0"], 1e-30, 1e-30, what="tiny delta keeps the state")
    reset = dict(c, delta=np.full_like(c["delta"], 60.0))
    y, hT = orc.scan(**reset)
    _close(hT, 60.0 * c["B"][:, -1, None, :] * c["x"][:, -1, :, None], 1e-12, what="large delta resets")


def check_decode_steps_equal_full(orc):
    """L successive L=1 calls with the state passed along equal one length-L call."""
    c = _rand_case(91, bsz=3, L=16, dim=4, N=4)
    y, hT = orc.scan(**c)
    h = c["h0"]
    ys = []
    for t in range(16):
        st = {k: (v[:, t: t + 1] if k in ("x", "delta", "B", "C", "z") else v) for k, v in c.items()}
        st["h0"] = h
        yt, h = orc.scan(**st)
        ys.append(yt)
    assert np.array_equal(np.concatenate(ys, axis=1), y)
    assert np.array_equal(h, hT)


def check_threads_do_not_change_results(orc):
    c = _rand_case(101, bsz=3, L=20, dim=7, N=4)
    y1, h1 = orc.scan(**c, threads=1)
    y8, h8 = orc.scan(**c, threads=8)
    assert np.array_equal(y1, y8) and np.array_equal(h1, h8)


ALL_CHECKS = [
    check_softplus_values,
    check_l1_by_hand,
    check_l2_n2_by_hand,
    check_A_zero_is_cumsum,
    check_constant_inputs_geometric,
    check_bruteforce_unrolled,
    check_assoc_twin,
    check_chunked_equals_full,
    check_causality,
    check_linearity,
    check_gate_and_readout_special_cases,
    check_delta_limits,
    check_decode_steps_equal_full,
    check_threads_do_not_change_results,
]
