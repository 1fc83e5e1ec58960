"""The CPU oracle against its pins (no GPU needed)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin, orc):
    pin(orc)


def test_oracle_uses_threads(orc):
    assert orc.num_threads() >= 1
