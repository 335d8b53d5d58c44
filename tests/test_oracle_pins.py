"""The CPU oracle against every pin (worked examples, closed forms, invariants,
brute force and library special cases).  CPU only."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
