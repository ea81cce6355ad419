"""The CPU oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle
from tests import oracle_pins as P


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", [p for p in P.ALL_PINS], ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_p2_metrics_reading():
    P.pin_p2_metrics_reading()
