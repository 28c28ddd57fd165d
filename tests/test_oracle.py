"""The CPU oracle against brute force, closed forms, invariants and the
format figures of the PerfXLLM page (§3.1).  CPU only."""

import pytest

import oracle.w4a16 as ora
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(ora)
