"""The oracle against its pins (closed forms, invariants, finite differences,
brute force, torch's CPU float64 routines, the page's recurrence)."""
import pytest

import oracle
from tests import oracle_checks as oc


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle)
