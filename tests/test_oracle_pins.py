"""The CPU oracle against its pins (exact rationals, 50-digit decimals, an
independent BLAS, brute force, closed forms, invariants, the pages' values)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def o():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.FAST, ids=lambda f: f.__name__)
def test_fast_pin(o, pin):
    pin(o)


@pytest.mark.slow
@pytest.mark.parametrize("pin", oracle_pins.SLOW, ids=lambda f: f.__name__)
def test_slow_pin(o, pin):
    pin(o)
