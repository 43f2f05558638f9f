"""The oracle against what the pages and mathematics fix (no GPU needed)."""
import ctypes

import pytest

import pins


@pytest.fixture(scope="module")
def L(oracle_lib):
    return pins.bind(ctypes.CDLL(oracle_lib.LIB_PATH))


@pytest.mark.parametrize("pin", pins.CORE_PINS, ids=lambda p: p.__name__)
def test_core_pin(L, pin):
    fails = pin(L)
    assert not fails, "\n".join(fails)


def test_rejects_out_of_definition_arguments(L):
    import numpy as np
    codes = np.zeros((2, 32), np.uint8)
    scales = np.ones((2, 1), np.float32)
    x = np.zeros(64, np.float64)
    y = np.zeros(2, np.float64)
    p = pins._p
    assert L.oracle_qmatvec(p(codes), p(scales), 3, 64, 2, 64, p(x), p(y)) == -1   # bits
    assert L.oracle_qmatvec(p(codes), p(scales), 4, 48, 2, 64, p(x), p(y)) == -1   # group
    assert L.oracle_qmatvec(p(codes), p(scales), 4, 64, 0, 64, p(x), p(y)) == -1   # rows
    assert L.oracle_qmatvec(None, p(scales), 4, 64, 2, 64, p(x), p(y)) == -1       # NULL
