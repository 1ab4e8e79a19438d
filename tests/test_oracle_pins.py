"""The CPU oracle against its pins (values printed on the pages, closed forms,
exact brute force, invariants, special cases and library routines)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)
