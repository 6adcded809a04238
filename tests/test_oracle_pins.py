"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import pytest

import oracle.gqe_oracle as orc
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(orc)
