"""The float64 oracle against the pins in oracle_pins.py (CPU only)."""
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle.mla_oracle)
