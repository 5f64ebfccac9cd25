"""The CPU oracle against brute force, closed forms, invariants, a library routine and
the pages' KV-size figures (no GPU needed)."""
import pytest

import oracle.attention as att
import oracle.footprint as fp
import oracle.kvq8 as q8
import oracle.proj as pj
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(att)


def test_footprint():
    P.pin_footprint(att, fp)


@pytest.mark.parametrize("pin", P.Q8_PINS, ids=lambda f: f.__name__)
def test_q8_pin(pin):
    pin(q8)


@pytest.mark.parametrize("pin", P.Q8_ATT_PINS, ids=lambda f: f.__name__)
def test_q8_att_pin(pin):
    pin(att, q8)


def test_q8_row_bytes():
    P.pin_q8_row_bytes(q8, fp)


@pytest.mark.parametrize("pin", P.PROJ_PINS, ids=lambda f: f.__name__)
def test_proj_pin(pin):
    pin(pj)


@pytest.mark.parametrize("pin", P.PROJ_ATT_PINS, ids=lambda f: f.__name__)
def test_proj_att_pin(pin):
    pin(att, pj)
