"""The oracle against its pins (CPU only)."""
import pytest

from oracle import oracle as orc
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(orc.load())
