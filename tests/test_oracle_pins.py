"""The oracle against its pins (CPU only)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def o():
    oracle.build()           # always test the oracle built from its source
    return oracle.Oracle()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)
