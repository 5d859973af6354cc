"""The CPU oracle against brute force, scipy, closed forms and invariants (no GPU)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def o():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)
