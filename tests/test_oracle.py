"""CPU-only: the oracle against its pins (library routines, brute force,
closed forms and invariants of the method). See tests/oracle_pins.py."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin()
