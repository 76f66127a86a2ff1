"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import pins


@pytest.fixture(scope="module")
def fwd(oracle_mod):
    return oracle_mod.forward


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(fwd, pin):
    pin(fwd)
