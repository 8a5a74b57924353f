"""The oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return oracle._get()


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__[6:])
def test_oracle_pin(check, lib):
    check(lib)
