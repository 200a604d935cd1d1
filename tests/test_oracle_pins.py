"""CPU tests: the oracle against its pins (closed forms, invariants, brute
force, witnesses, worked examples).  No GPU involved."""
import numpy as np
import pytest

import oracle
from pins import ALL_PINS


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, lib):
    pin(lib)


def test_rejects_bad_arguments(lib):
    q = np.zeros((1, 1, 4, 8))
    with pytest.raises(RuntimeError):
        oracle.attention(q, q, q, 1.0, False, rows=[4], lib=lib)  # row out of range
    with pytest.raises(RuntimeError):
        oracle.attention_online(q, q, q, 1.0, False, 0, 4, lib=lib)  # empty tile


def test_threads_reported(lib):
    assert oracle.threads(lib) >= 1
