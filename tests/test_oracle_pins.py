"""The CPU oracle against its pins (hand-derived examples, closed forms, brute
force, library reductions).  CPU only."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: getattr(p, "__name__", "lambda"))
def test_pin(pin):
    pin()
