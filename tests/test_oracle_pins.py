"""Run every oracle pin (tests/oracle_pins.py) on the oracle as built."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(olib, pin):
    pin(olib)
