"""The oracle against its pins (values the pages print, textbook values, closed forms,
brute force and invariants). CPU only."""
import pytest

import oracle_pins
from oracle import moe_oracle


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(moe_oracle)
