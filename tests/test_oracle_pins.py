"""The CPU oracle against its pins (fixtures, closed forms, brute force, invariants)."""
import pytest

import oracle
import pinlib


@pytest.mark.parametrize("pin", pinlib.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.load())
