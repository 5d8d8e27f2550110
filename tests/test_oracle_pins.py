"""The fp64 oracle against its pins (CPU only)."""

import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    if pin.__name__.startswith("pin_brute") and oracle_pins.mpmath is None:
        pytest.skip("mpmath not importable")
    pin(oracle)
