"""The CPU oracle against the pages' printed values, closed forms, library
routines and invariants (no GPU)."""

import pytest

from oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=[c.__name__ for c in ALL_CHECKS])
def test_oracle_pin(check):
    check()
