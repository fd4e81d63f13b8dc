"""The gfx950 rates the forward kernel's design rests on, measured by the
probes in tests/hw_probes/ (built by __graft_entry__.build()):

- a lone wave issues at most one VALU instruction every ~4 cycles, dependent
  or not, while a SIMD runs the instructions of two waves in about half that
  time each;
- a fused multiply-add whose sources share the accumulator's VGPR bank, or
  takes a scalar (SGPR) or DPP-broadcast operand, costs the SIMD about twice
  a plain one; a transcendental about four times a multiply;
- LDS reads of 16 bytes per lane move about twice the bytes of two-dword
  reads, and writes move fewer bytes per ns than reads;
- a wave's plain FMA stream keeps its rate when the other wave of its SIMD
  runs FMAs or transcendentals; a DPP-operand stream loses some of it to a
  transcendental stream.

Only relations with wide margins are asserted (the absolute rates depend on
the clock under load); the measured table is printed.
"""
from __future__ import annotations

import os
import subprocess

import pytest
import torch

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP GPU"),
]

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hw_probes", "bin")


def _run(name):
    exe = os.path.join(BIN, name)
    if not os.path.exists(exe):
        pytest.fail(f"{exe} missing: run __graft_entry__.build() first")
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120, check=True).stdout
    print(out)
    rates = {}
    for line in out.splitlines():
        case, n, v = line.split()
        rates[(case, int(n))] = float(v)
    return rates


def test_valu_issue_costs():
    r = _run("valu_issue")
    fma1, fma2 = r[("fma", 1)], r[("fma", 2)]
    assert fma2 < 0.7 * fma1, "two waves per SIMD should overlap their VALU instructions"
    for w in (2, 4):
        base = r[("fma", w)]
        assert r[("fma_bank_conflict", w)] > 1.4 * base
        assert r[("fma_sgpr", w)] > 1.4 * base
        assert r[("fma_dpp", w)] > 1.4 * base
        assert r[("exp", w)] > 2.5 * r[("mul", w)]
    # a lone wave pays nothing for dependences beyond its issue slot: one chain
    # of dependent FMAs runs at the rate of eight independent ones
    assert r[("fma_chain", 1)] < 1.2 * fma1
    assert r[("fma_dpp_chain", 1)] < 1.2 * r[("fma_dpp", 1)]


def test_lds_widths():
    r = _run("lds_rate")
    for w in (8, 16):
        assert r[("read_b128", w)] > 1.4 * r[("read_2x_b32", w)]
        assert r[("write_b128", w)] < r[("read_b128", w)]


def test_wave_pairs_on_one_simd():
    r = _run("wave_mix")
    assert r[("fma_with_fma", 1)] < 1.1 * r[("fma_alone", 1)]
    assert r[("fma_with_exp", 1)] < 1.1 * r[("fma_alone", 1)]
    assert r[("dppfma_with_exp", 1)] > 1.04 * r[("dppfma_alone", 1)]
