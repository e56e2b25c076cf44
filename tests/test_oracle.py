"""The CPU oracle against its pins (see oracle_pins.py for what each pin ties it to)."""
import pytest

from oracle import paged_attention as orc
from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(orc)
