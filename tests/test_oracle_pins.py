"""The fp64 oracle against closed forms, invariants, library routines, brute
force and the hand-worked golden example (see ``pins.py``)."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=[p.__name__ for p in pins.ALL_PINS])
def test_pin(pin):
    pin(oracle.get())
