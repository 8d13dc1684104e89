"""CPU: planted mistakes in the oracle (built with -DORACLE_MUTANT=k) must each fail at
least one pin — evidence that the pins would catch a plausible error in the oracle."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.mark.parametrize("k", sorted(oracle.MUTANTS), ids=lambda k: f"mutant{k}")
def test_mutant_is_caught(k):
    orc = oracle.mutant(k)
    caught = []
    for pin in PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError) as e:   # ValueError: the oracle rejected input
            caught.append(pin.__name__)
            break
    assert caught, f"mutant {k} ({oracle.MUTANTS[k]}) passed every pin"
