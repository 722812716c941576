"""The CPU oracle against its pins (worked example, brute force, library routine, closed forms,
invariances).  CPU only."""

import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()
