"""The CPU oracle against its pins (brute force, closed forms, worked
examples from the pages, exhaustive decoder checks).  No GPU needed."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)
