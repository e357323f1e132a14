"""The oracle agrees with brute force, torch SDPA (fp64), closed forms and invariants."""
import pytest

import pinlib


@pytest.mark.parametrize("check", pinlib.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(check):
    check()
