"""The oracle against its pins (CPU only)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)
