"""The CPU oracle against its pins (hand-worked fixture, closed forms, brute
force, rebuild equivalence, decimal reference, chi-square)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def lib():
    oracle.build(force=False)
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)
