"""The CPU oracle against its pins (no GPU needed)."""

import pytest

from oracle import oracle as O

from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def lib():
    return O.load()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(lib, pin):
    pin(lib)
