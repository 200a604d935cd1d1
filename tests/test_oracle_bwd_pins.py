"""CPU tests: the oracle's backward pass against its pins (finite differences
of the forward oracle, closed forms, sum rules, an autograd witness)."""
import numpy as np
import pytest

import oracle
from pins_bwd import ALL_BWD_PINS


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_BWD_PINS, ids=lambda p: p.__name__)
def test_bwd_pin(pin, lib):
    pin(lib)


def test_bwd_rejects_bad_arguments(lib):
    x = np.zeros((1, 1, 4, 8))
    with pytest.raises(RuntimeError):
        oracle.attention_bwd(x, x, x, x, 1.0, False, qrows=[4], lib=lib)
    with pytest.raises(RuntimeError):
        oracle.attention_bwd(x, x, x, x, 1.0, True, krows=[-1], lib=lib)
