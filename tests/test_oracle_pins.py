"""The float64 oracle against facts the mathematics fixes (see tests/pins.py)."""
import pytest

from oracle import oracle
from tests import pins


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("name", sorted(pins.PINS))
def test_pin(lib, name):
    err = pins.PINS[name](lib)
    assert err <= pins.PIN_TOL[name], f"{name}: {err}"


def test_rejects_bad_arguments(lib):
    import numpy as np
    q = np.zeros((4, 1, 2), np.float32)
    v = np.zeros((4, 3, 2), np.float32)   # Hv=3 not a multiple of Hk=2 below
    g = np.zeros((4, 3), np.float32)
    with pytest.raises(ValueError):
        oracle.reference(np.zeros((4, 2, 2), np.float32), np.zeros((4, 2, 2), np.float32),
                         v, g, g, [4], lib=lib)
    with pytest.raises(ValueError):      # lengths do not sum to T
        oracle.reference(q, q, np.zeros((4, 1, 2), np.float32), g[:, :1], g[:, :1], [3], lib=lib)
