"""The CPU oracle against brute force, closed forms, invariants, a library routine and
the pages' KV-size figures (no GPU needed)."""
import pytest

import oracle.attention as att
import oracle.footprint as fp
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(att)


def test_footprint():
    P.pin_footprint(att, fp)
