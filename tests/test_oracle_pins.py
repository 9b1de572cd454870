"""The CPU oracle against its pins (hand-worked fixtures, closed forms, brute
force, exact rationals, the lookup-table cross-check and invariants)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()
