"""The CPU oracle against its pins (closed forms, printed values, brute force,
library routines). CPU only."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("name", sorted(oracle_pins.ALL_PINS))
def test_pin(orc, name):
    oracle_pins.ALL_PINS[name](orc)
