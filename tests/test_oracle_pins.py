"""The CPU oracle against its pins (hand-worked fixtures, closed forms,
invariants, library routines on special cases, fp64 brute force)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, orc):
    pin(orc)
