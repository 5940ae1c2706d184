"""The oracle against what the pages and the mathematics fix (CPU only)."""

import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()
