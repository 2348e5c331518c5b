"""The fp64 oracle against what the pages and the mathematics fix (no GPU needed)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(orc, check):
    check(orc)
