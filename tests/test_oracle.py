"""The CPU oracle against closed forms, brute force, a library routine, invariants and the
pages' worked examples (see ``oracle_pins.py``)."""
import pytest

from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin()
