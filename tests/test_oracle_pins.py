"""CPU reference pinned to the pages and to mathematics (runs without a GPU)."""
import pytest

from tests import pins


@pytest.mark.parametrize("check", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
