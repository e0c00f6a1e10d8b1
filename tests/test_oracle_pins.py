"""The CPU oracle against facts that do not come from itself (see tests/oracle_pins.py)."""

import pytest

import oracle
from oracle_pins import PINS


@pytest.mark.parametrize("name", sorted(PINS))
def test_oracle_pin(name):
    PINS[name](oracle)
