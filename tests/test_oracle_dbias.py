"""Pins of the oracle's bias gradient (column sums of the output gradient,
fp32) -- the gradient of the biased linears in the training loop of "CPU
Overhead of te.Linear FP8 Layers".  Checked against closed forms, exact
integer cases, Python's correctly rounded math.fsum (an independent exact
summation), and row-permutation invariance."""
import math

import numpy as np
import pytest

import oracle


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, for values that are exact in bf16."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    assert not (b & 0xFFFF).any(), "test value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def test_all_ones_is_the_row_count():
    for rows, cols in ((1, 1), (7, 3), (300, 16), (8192, 4)):
        x = _bf16_bits(np.ones((rows, cols), np.float32))
        np.testing.assert_array_equal(oracle.dbias(x), np.full(cols, rows, np.float32))


def test_column_index_values():
    rows, cols = 37, 50
    x = np.tile(np.arange(1, cols + 1, dtype=np.float32), (rows, 1))
    np.testing.assert_array_equal(oracle.dbias(_bf16_bits(x)), rows * np.arange(1, cols + 1, dtype=np.float32))
    np.testing.assert_array_equal(oracle.dbias(x), rows * np.arange(1, cols + 1, dtype=np.float32))


def test_alternating_signs_cancel():
    rows, cols = 64, 9
    x = np.where((np.arange(rows)[:, None] % 2) == 0, 3.0, -3.0).astype(np.float32) * np.ones((1, cols), np.float32)
    np.testing.assert_array_equal(oracle.dbias(_bf16_bits(x)), np.zeros(cols, np.float32))
    x[-1] = 5.0                                       # last row (odd) now +5 instead of -3
    np.testing.assert_array_equal(oracle.dbias(x), np.full(cols, 8.0, np.float32))


def test_bf16_random_against_fsum():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((300, 77)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)       # truncate to bf16 values
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    want = np.array([np.float32(math.fsum(vals[:, c].astype(np.float64))) for c in range(77)])
    np.testing.assert_array_equal(oracle.dbias(bits), want)


def test_fp32_grid_values_against_fsum():
    rng = np.random.default_rng(4)
    x = (np.round(rng.standard_normal((513, 40)) * 1024) / 1024).astype(np.float32)
    want = np.array([np.float32(math.fsum(x[:, c].astype(np.float64))) for c in range(40)])
    np.testing.assert_array_equal(oracle.dbias(x), want)


def test_row_permutation_invariance():
    rng = np.random.default_rng(5)
    bits = (rng.standard_normal((200, 33)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    perm = rng.permutation(200)
    np.testing.assert_array_equal(oracle.dbias(bits), oracle.dbias(np.ascontiguousarray(bits[perm])))


def test_empty_and_bad_arguments():
    np.testing.assert_array_equal(oracle.dbias(np.zeros((0, 5), np.uint16)), np.zeros(5, np.float32))
    assert oracle.dbias(np.zeros((4, 0), np.float32)).shape == (0,)
    with pytest.raises(TypeError):
        oracle.dbias(np.zeros((2, 2), np.float64))
