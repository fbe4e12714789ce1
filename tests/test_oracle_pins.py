"""The fp64 oracle against closed forms, library routines, invariants and brute
force (CPU only)."""

import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)
