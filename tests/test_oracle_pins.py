"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle_checks


@pytest.mark.parametrize("check", oracle_checks.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check()
