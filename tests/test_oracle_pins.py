"""The fp64 oracle against hand-worked values, brute force, torch SDPA, closed forms and invariants."""
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle)


@pytest.mark.parametrize("check", pins.PROLOGUE_CHECKS, ids=lambda f: f.__name__)
def test_prologue_pin(check):
    check(oracle.prologue)


@pytest.mark.parametrize("check", pins.GDN_CHECKS, ids=lambda f: f.__name__)
def test_gated_delta_pin(check):
    check(oracle.linear_attention)
