"""The fp64 oracle against closed forms, a decimal brute force, the
MicroAttention identities and the hand-derived worked example (CPU only)."""

import pytest

import oracle
from oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)
