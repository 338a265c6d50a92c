"""The CPU oracle against closed forms, library routines, invariants and brute force (no GPU)."""
import pytest

from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(oracle_mod, pin):
    pin()
