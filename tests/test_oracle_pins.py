"""The oracle against closed forms, library routines, brute force and
invariants (CPU only)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
