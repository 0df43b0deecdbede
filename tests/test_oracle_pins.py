"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_rejects_bad_arguments(lib):
    import numpy as np
    q = np.zeros((2, 2, 4), np.float32)
    pool = np.zeros((2, 16, 1, 4), np.float32)
    with pytest.raises(ValueError):  # context longer than the page table
        oracle.decode(q, pool, pool, np.zeros((2, 1), np.int32), [4, 17], 1.0, lib=lib)
    with pytest.raises(ValueError):  # context 0
        oracle.decode(q, pool, pool, np.zeros((2, 1), np.int32), [0, 1], 1.0, lib=lib)
    with pytest.raises(ValueError):  # row outside the chunk
        oracle.prefill(q, pool, pool, np.zeros(1, np.int32), 0, 1.0, rows=[2], lib=lib)
