"""The CPU oracle against its pins (hand-derived example, closed forms,
invariants, brute force and an independent table-driven implementation)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("name,check", pins.ALL_CHECKS, ids=[n for n, _ in pins.ALL_CHECKS])
def test_pin(lib, name, check):
    check(lib)
