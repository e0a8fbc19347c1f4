"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle_pins
import oracle_pins_unet


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS + oracle_pins_unet.ALL_PINS,
                         ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()
