"""The oracle against its pins (closed forms, invariants, brute force)."""
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, lib):
    pin(lib)
