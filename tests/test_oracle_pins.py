"""CPU: the f64 oracle against its pins (closed forms, a library attention routine,
exhaustive dtype decoding, invariants, brute-force causality, printed causal extents)."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle._load())
