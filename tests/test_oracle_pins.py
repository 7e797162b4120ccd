"""The CPU oracle against its pins (hand-worked fixtures, brute force, closed forms,
invariants).  CPU only."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, lib):
    pin(lib)
