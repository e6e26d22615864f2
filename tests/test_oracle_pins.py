"""The oracle against its pins (CPU only)."""
import pytest

from oracle import Oracle
from tests.oracle_pins import ALL_PINS, SWEEP_PINS


@pytest.fixture(scope="module")
def orc():
    return Oracle()


@pytest.mark.parametrize("pin", ALL_PINS + SWEEP_PINS,
                         ids=[p.__name__ for p in ALL_PINS + SWEEP_PINS])
def test_pin(orc, pin):
    pin(orc)
