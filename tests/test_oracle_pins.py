"""The FP64 oracle against facts it does not define itself (see oracle_pins for the list)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_finite_differences_without_norm(oracle_lib):
    oracle_pins.pin_finite_differences(oracle_lib, l2norm=False, seed=21)
