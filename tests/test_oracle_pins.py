"""The fp64 oracle against what the pages and mathematics fix (CPU only)."""
import pytest

from tests import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(ora, check):
    check(ora)
