"""The CPU oracle against what fixes it from outside (CPU only)."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin, orc):
    pin(orc)
