"""The oracle against its pins (CPU only)."""
import pytest

from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(oracle_mod, pin):
    pin(oracle_mod)
