"""The FP64 oracle against its pins (CPU only)."""
import pytest

import oracle.attention as oracle_mod
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle_mod)
