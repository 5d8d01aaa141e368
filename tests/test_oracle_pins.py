"""The fp64 oracle against closed forms, brute force, identities and finite differences."""

import pytest

import oracle_pins
from oracle import coda_oracle as O


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(O)
