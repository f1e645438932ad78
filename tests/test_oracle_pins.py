"""The CPU oracle against its pins (see oracle_pins.py for what each fixes)."""
import pytest

from oracle import kvq_oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(kvq_oracle)
