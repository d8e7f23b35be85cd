"""Each planted mistake in the oracle must be caught by at least one pin.

The mistakes are compiled into separate builds of oracle.c (-DORACLE_MUTANT=k)
on the CPU; the real oracle is untouched.
"""

import pytest

import oracle
import pins


@pytest.mark.parametrize("mutant", sorted(pins.MUTANTS), ids=lambda k: pins.MUTANTS[k])
def test_mutant_is_caught(mutant):
    oracle.build(mutant, force=False)
    failed = pins.failing_pins(mutant)
    assert failed, f"planted mistake '{pins.MUTANTS[mutant]}' passed every pin"
