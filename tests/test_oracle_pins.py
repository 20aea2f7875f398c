"""The oracle against its pins (CPU): see oracle_pins.py for what each pin fixes and why."""
import pytest

from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)
