"""The CPU oracle against its pins (no GPU needed)."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(oracle)


def test_round_to_storage_ties_to_even():
    import numpy as np
    # bf16: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> ties to even (1.0)
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.0, 65504.0])
    assert oracle.round_to_storage(x, "bf16").tolist() == [0x3F80, 0x3F82, 0xC000, 0x4780]
    assert oracle.round_to_storage(np.array([1 + 2 ** -11]), "f16").tolist() == [0x3C00]
