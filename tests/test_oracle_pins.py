"""The fp64 oracle against what the pages and the mathematics fix."""

import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, pin):
    pin(0)
