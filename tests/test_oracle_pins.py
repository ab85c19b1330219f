"""The fp64 oracle against its pins (values the pages print, closed forms,
exact enumeration, chi-square tests, library cross-checks)."""
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def o():
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)
