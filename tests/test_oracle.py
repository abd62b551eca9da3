"""The fp64 oracle against its pins (no GPU)."""
import pytest

from tests.oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=[c.__name__ for c in ALL_CHECKS])
def test_oracle_pin(check):
    check()
