"""The fp64 oracle against values the pages and the mathematics fix (CPU)."""
import pytest

from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
