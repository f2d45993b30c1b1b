"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import pytest

from oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=[c.__name__ for c in ALL_CHECKS])
def test_oracle_pin(orc, check):
    check(orc)
