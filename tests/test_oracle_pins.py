"""The oracle against exact brute force, closed forms, invariants and special cases."""
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.default())
