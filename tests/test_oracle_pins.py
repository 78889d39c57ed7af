"""Every pin check of tests/oracle_pins.py, run on the CPU oracle."""
import pytest

import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle_mod, check):
    check(oracle_mod)
