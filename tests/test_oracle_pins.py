"""The oracle against what the pages and the mathematics fix (CPU only)."""

import pytest

from tests import oracle_pins as P

PINS = [name for name in dir(P) if name.startswith("pin_")]


@pytest.mark.parametrize("name", PINS)
def test_pin(name):
    getattr(P, name)()
