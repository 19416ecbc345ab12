"""The CPU oracle against values printed on the pages, closed forms and
invariants (all on the CPU; see ``tests/pins.py`` for each pin's source)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, oracle_default):
    pin(oracle_default)
