"""The CPU oracle against its pins (worked groups, library bf16 conversion,
closed forms, invariants, special cases, scalar brute force).  No GPU."""
import pytest

from tests import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()
