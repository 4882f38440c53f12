"""The fp64 oracle against its pins (closed forms, brute force, invariants,
hand-worked examples); see pins.py for what each pin fixes."""
import pytest

from pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)

