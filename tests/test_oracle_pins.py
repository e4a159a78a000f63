"""The CPU oracle against its pins (formats, fixtures, brute force, closed forms,
invariants). CPU only."""

import pytest

import pins
from oracle import far_oracle


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(far_oracle)
