"""The fp64 oracle against its closed-form pins (CPU only)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, check):
    check(orc)


def test_oracle_is_not_a_mutant(orc):
    assert orc.mutant == 0
