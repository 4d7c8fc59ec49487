"""The CPU oracle against its pins (no GPU)."""

import functools

import numpy as np
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def gemm():
    oracle.build()
    return functools.partial(oracle.gemm, threads=4)


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(pin, gemm):
    pin(gemm)


def test_thread_count_invariance():
    from dense_fp32_gemm_row_amd.workloads import make_inputs

    A, B = make_inputs(96, 80, 513, "uniform", seed=3)
    one = oracle.gemm(A, B, threads=1)
    many = oracle.gemm(A, B, threads=8)
    assert np.array_equal(one.view(np.uint32), many.view(np.uint32))


def test_invalid_arguments_rejected():
    lib = oracle.load()
    # lda < K
    rc = lib.oracle_gemm(2, 2, 3, None, 2, None, 2, None, 2, None, 2, None, 2, 1)
    assert rc == -1
    # rows NULL but nrows != M
    rc = lib.oracle_gemm(2, 2, 0, None, 1, None, 2, None, 1, None, 2, None, 2, 1)
    assert rc == -1
