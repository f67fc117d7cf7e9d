"""The KV-append oracle against its pins (nearest-even rounding, the complex
form of RoPE, closed forms, invariants, slots computed from the table)."""
import pytest

import oracle
from tests import oracle_append_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_append_pins.PINS, ids=lambda f: f.__name__)
def test_pin(pin, lib):
    pin(lib)
