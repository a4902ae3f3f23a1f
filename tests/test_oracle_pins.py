"""The CPU oracle against its pins (closed forms, brute force, library
routines, hand-worked examples): runs without a GPU."""
import pytest

from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle, pin):
    pin(oracle)
