"""The CPU oracle against its pins (hand derivations, f64 brute force, closed forms,
invariants, an exact-rational emulator). No GPU needed."""

import pytest

import oracle_pins
from oracle import oracle as O


@pytest.fixture(scope="module")
def orc():
    O.build(force=False)
    return O.get()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)
