"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import pytest

from oracle import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
