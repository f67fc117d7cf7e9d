"""The chunked-prefill oracle against its pins (masked torch SDPA, the decode
step at each chunk's last row, closed forms, re-chunking)."""
import pytest

import oracle
from tests import oracle_prefill_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_prefill_pins.PINS, ids=lambda f: f.__name__)
def test_pin(pin, lib):
    pin(lib)
