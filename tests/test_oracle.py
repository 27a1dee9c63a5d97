"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle_pins  # noqa: E402


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
