"""The fp64 oracle against what the pages, the OCP MX spec and mathematics fix (CPU)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
