"""The oracle against its pins (closed forms, brute force, library routines, page figures)."""
import pytest

from tests import oracle_checks as oc


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
