"""The CPU oracle against facts fixed outside it (closed forms, library
routines, invariants, brute force, hand-derived golden counts)."""
import pytest

from pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=[c.__name__ for c in ALL_CHECKS])
def test_oracle_pin(check):
    check(None)
