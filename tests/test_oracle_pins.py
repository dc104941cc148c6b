"""The CPU oracle checked against facts outside itself (no GPU needed)."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    ok, detail = pin()
    assert ok, detail
