"""The CPU oracle against its pins (hand-worked cases, brute force, closed
forms, special cases and invariants); see oracle_pins.py."""
import pytest

import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(orc, check):
    check(orc)
