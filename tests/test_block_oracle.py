"""The RMSNorm + residual neighbours of the oracle against their pins (no GPU)."""
import pytest

from tests.block_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=[c.__name__ for c in ALL_CHECKS])
def test_block_pin(check):
    check()
