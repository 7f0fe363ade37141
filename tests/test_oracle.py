"""The fp64 oracle against the pages' worked examples, closed forms, torch's
attention routine and a pure-Python brute force (all on the CPU)."""
import pytest

import oracle.mla_direct as O
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(O)
