"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import pin_checks


@pytest.mark.parametrize("check", pin_checks.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()
