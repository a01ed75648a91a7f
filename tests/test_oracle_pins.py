"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
