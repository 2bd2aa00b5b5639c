"""The CPU oracle against its pins (closed forms, worked example, FD, autograd, invariants)."""

import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
