"""The oracle against its pins (CPU only).  See oracle_pins.py for what each
check ties the oracle to."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)
