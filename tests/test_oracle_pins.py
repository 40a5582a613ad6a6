"""The CPU oracle against its pins (closed forms, library routines, published
values, brute force, invariants).  See tests/oracle_pins.py for the checks."""
import pytest

import oracle
import oracle_pins as pins


@pytest.fixture(scope="module")
def o():
    oracle.build(force=False)
    return oracle.default()


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__[6:])
def test_pin(o, check):
    check(o)
