"""The fp64 oracle against closed forms, golden hand-stepped values, torch.nn.LSTM / nn.RNN in
float64, and invariants (see tests/oracle_pins.py)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
