"""CPU pins of the oracle (no GPU): each check compares the oracle with something it did not
compute itself; see tests/oracle_pins.py for what each one fixes."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
