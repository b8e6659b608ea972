"""The CPU oracle against its pins (brute force, closed forms, invariants,
library routines, finite differences)."""
import pytest

import oracle
from pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(oracle)
