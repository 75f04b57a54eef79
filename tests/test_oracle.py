"""The fp64 oracle against its pins (see oracle_pins.py for what pins what)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(lib, pin):
    pin(lib)


def test_oracle_rejects_bad_arguments(lib):
    import numpy as np
    z = np.zeros((1, 1, 4, 8), np.uint16)
    with pytest.raises(TypeError):
        oracle.attention_fwd(z.astype(np.float32), z, z, scale=1.0, causal=False, dtype="f16", lib=lib)
    with pytest.raises(RuntimeError):
        oracle.attention_rows(z, z, z, np.array([4]), scale=1.0, causal=False, dtype="f16", lib=lib)
