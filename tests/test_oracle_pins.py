"""The CPU oracle against its pins (hand-worked blocks, exhaustive bit-field
enumerations, closed forms, an exact-rational brute force, library routines).
See oracle_pins.py for what each pin fixes and where the pages define it."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)
