"""CPU tests: the oracle's variable-length attention against its pins."""
import numpy as np
import pytest

import oracle
from pins_varlen import ALL_VARLEN_PINS


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_VARLEN_PINS, ids=lambda p: p.__name__)
def test_varlen_pin(pin, lib):
    pin(lib)


def test_varlen_rejects_bad_offsets(lib):
    x = np.zeros((1, 4, 8))
    with pytest.raises(ValueError):
        oracle.attention_varlen(x, x, x, [0, 3], [0, 4], 1.0, False, lib=lib)
    with pytest.raises(ValueError):
        oracle.attention_varlen(x, x, x, [0, 3, 2, 4], [0, 1, 2, 4], 1.0, False, lib=lib)
