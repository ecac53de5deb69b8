"""The oracle agrees with every fact the pages and the mathematics fix."""
import pytest

import oracle.ternary as o
from conftest import read_golden
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(o, read_golden)
