"""The oracle against facts other than itself (CPU only)."""
import pytest

from oracle import oracle as orc
from tests import oracle_pins as pins


@pytest.fixture(scope="module")
def lib():
    return orc.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, lib):
    pin(lib)
