"""The fp64 oracle against closed forms, brute force and invariants that do
not come from the oracle itself (see oracle_pins for what each one states)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)
