"""The CPU oracle against facts fixed outside it (formats, worked cases, closed
forms, invariants, brute force).  See oracle_pins.py for what pins what."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[p.__name__ for p in P.ALL_PINS])
def test_pin(orc, pin):
    pin()


def test_every_pin_is_collected():
    names = {n for n in dir(P) if n.startswith("pin_") and callable(getattr(P, n))}
    assert names == {p.__name__ for p in P.ALL_PINS}
