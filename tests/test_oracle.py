"""CPU oracle against its pins (printed examples, closed forms, invariants, brute force)."""
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=[p.__name__ for p in pins.ALL_PINS])
def test_pin(pin):
    pin()
