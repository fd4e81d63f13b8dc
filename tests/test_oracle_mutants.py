"""Every deliberately broken oracle build fails at least one pin (CPU only).

Each mutant is a plausible slip planted in the oracle source behind
ORACLE_MUTANT=k (sign of A, dropped bias, swapped B/C, read-before-update,
skip term without x, sigmoid for SiLU, ...).  If a mutant passed every pin,
the pins would not be pinning that part of the oracle.
"""
import os

import pytest

import oracle
from tests import oracle_pins

MUTANTS = list(range(1, 15))  # forward mutants; 15-18: backward (test_oracle_bwd.py); 19-20: conv prologue (test_oracle_conv.py); 21-22: SSD (test_oracle_ssd.py); 23-25: gated linear attention (test_oracle_gla.py); 26-27: zero-order hold (test_oracle_zoh.py); 28-29: zero-order-hold backward (test_oracle_bwd.py)


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("oracle_mutants"))


@pytest.mark.parametrize("k", MUTANTS)
def test_mutant_is_caught(k, mutant_dir):
    path = oracle.build(mutant=k, out_dir=mutant_dir)
    orc = oracle.Oracle(path)
    assert orc.mutant == k
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(orc)
        except AssertionError:
            failed.append(check.__name__)
        except (FloatingPointError, ValueError, RuntimeError):
            failed.append(check.__name__)
    assert failed, f"mutant {k} passed every pin"
