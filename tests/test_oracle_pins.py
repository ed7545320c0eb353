"""The CPU oracle checked against values and properties fixed by the pages and by
mathematics (see tests/oracle_pins.py for each pin and its citation)."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
