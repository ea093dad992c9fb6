"""The fp64 attention oracle against closed forms, 50-digit brute force, torch's CPU float64
attention, invariants and the blockwise recurrences of Algorithm 1 (see oracle_pins.py)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def lib():
    oracle.build(force=False)
    return oracle._load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)
