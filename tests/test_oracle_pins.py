"""The CPU oracle against what the pages and the mathematics fix (no GPU needed)."""
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def O():
    return oracle.default()


@pytest.mark.parametrize("check", pins.ALL, ids=lambda f: f.__name__)
def test_pin(O, check):
    check(O)
