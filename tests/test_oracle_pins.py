"""Run every oracle pin on the real oracle (CPU only)."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.reference)
