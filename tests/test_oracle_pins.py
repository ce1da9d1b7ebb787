"""The CPU oracle against brute force, closed forms, library routines and the
page's configuration table (no GPU needed)."""
import pytest

from oracle import moe_oracle
from pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(moe_oracle)
