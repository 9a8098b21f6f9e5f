"""The CPU oracle against its pins (brute force, library routines, closed forms, a hand-worked example)."""
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle, pin):
    pin(oracle)
