"""Pins of the oracle's producer-fused cast: the toy block's elementwise
producers of "CPU Overhead of te.Linear FP8 Layers" (x = shift * x / scale
followed by nan_to_num, and the residual add), rounded to bf16.  Checked
against torch's own CPU bf16 arithmetic (an independent implementation of the
same operations), closed forms, and the already pinned cast oracle."""
import numpy as np
import pytest
import torch

import oracle


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _rand_bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16)


def _torch_modulate(a, x, b):
    y = (a.float() * x.float() / b.float()).to(torch.bfloat16)
    return torch.nan_to_num(y, nan=0.0, posinf=0.0, neginf=0.0)


def test_modulate_against_torch():
    a, x, b = _rand_bf16((96, 80), 1), _rand_bf16((96, 80), 2), _rand_bf16((96, 80), 3, 0.5)
    y, *_ = oracle.produce_cast(oracle.PROD_MODULATE, _bits(x), _bits(a), _bits(b), 1.0, oracle.E4M3)
    np.testing.assert_array_equal(y, _bits(_torch_modulate(a, x, b)))


def test_add_against_torch_including_nan():
    x, a = _rand_bf16((64, 48), 4), _rand_bf16((64, 48), 5, 100.0)
    x[0, 0] = float("nan")
    a[1, 1] = float("inf")
    x[2, 2] = float("-inf")
    a[2, 2] = float("inf")                        # -inf + inf = NaN
    y, *_ = oracle.produce_cast(oracle.PROD_ADD, _bits(x), _bits(a), None, 1.0, oracle.E5M2)
    want = x + a                                  # torch CPU: fp32 add, round to nearest even
    nan = torch.isnan(want).numpy()
    # torch's NaN bit pattern depends on its code path; the oracle writes 0x7FC0
    np.testing.assert_array_equal(y[~nan], _bits(want)[~nan])
    assert (y[nan] == 0x7FC0).all() and nan[0, 0] and nan[2, 2]
    assert y[1, 1] == 0x7F80


def test_add2_against_torch_including_nan():
    """Two residual terms: torch adds them one after the other, rounding each
    sum to bf16."""
    x, a, b = _rand_bf16((64, 48), 12), _rand_bf16((64, 48), 13, 10.0), _rand_bf16((64, 48), 14, 0.01)
    x[0, 0] = float("nan")
    a[1, 1] = float("inf")
    b[2, 2] = float("-inf")
    a[3, 3] = float("inf")
    b[3, 3] = float("-inf")                       # inf + -inf = NaN at the second add
    y, *_ = oracle.produce_cast(oracle.PROD_ADD2, _bits(x), _bits(a), _bits(b), 1.0, oracle.E4M3)
    want = (x + a) + b
    nan = torch.isnan(want).numpy()
    np.testing.assert_array_equal(y[~nan], _bits(want)[~nan])
    assert (y[nan] == 0x7FC0).all() and nan[0, 0] and nan[3, 3]
    assert y[1, 1] == 0x7F80 and y[2, 2] == 0xFF80


def test_add2_rounds_twice():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 and rounds to even (1); adding
    # 2^-8 again gives 1 again.  One rounding of the exact sum 1 + 2^-7 would
    # give 1 + 2^-7 (0x3F81).
    one = torch.ones(16, 16, dtype=torch.bfloat16)
    e = torch.full((16, 16), 2.0 ** -8, dtype=torch.bfloat16)
    y, *_ = oracle.produce_cast(oracle.PROD_ADD2, _bits(one), _bits(e), _bits(e), 1.0, oracle.E4M3)
    assert (y == 0x3F80).all()
    y, *_ = oracle.produce_cast(oracle.PROD_ADD, _bits(one), _bits(e + e), None, 1.0, oracle.E4M3)
    assert (y == 0x3F81).all()


def test_strided_views_match_torch():
    # shift and scale are column slices of the modulation linear's output,
    # the residual term a column slice of the qkv output.
    mod = _rand_bf16((64, 3 * 32), 6)
    x = _rand_bf16((64, 32), 7)
    shift, scale = mod[:, :32], mod[:, 32:64]
    mb = mod.view(torch.int16).numpy().view(np.uint16)      # [64, 96] bits, row stride 96
    y, *_ = oracle.produce_cast(oracle.PROD_MODULATE, _bits(x), mb[:, :32], mb[:, 32:64], 1.0,
                                oracle.E4M3)
    np.testing.assert_array_equal(y, _bits(_torch_modulate(shift, x, scale)))
    y, *_ = oracle.produce_cast(oracle.PROD_ADD, _bits(x), mb[:, 64:96], None, 1.0, oracle.E4M3)
    np.testing.assert_array_equal(y, _bits(x + mod[:, 64:96]))
    y, *_ = oracle.produce_cast(oracle.PROD_ADD2, _bits(x), mb[:, 64:96], mb[:, :32], 1.0,
                                oracle.E4M3)
    np.testing.assert_array_equal(y, _bits((x + mod[:, 64:96]) + mod[:, :32]))


def test_modulate_closed_forms():
    x = _rand_bf16((32, 16), 8)
    a = _rand_bf16((32, 16), 9)
    a[a == 0] = 1.0
    # b == a: the product of two bf16 values is exact in fp32, so a*x/a == x
    y, *_ = oracle.produce_cast(oracle.PROD_MODULATE, _bits(x), _bits(a), _bits(a), 1.0, oracle.E4M3)
    np.testing.assert_array_equal(y, _bits(x))
    # division by zero and 0/0 -> +0 (nan_to_num)
    z = torch.zeros(32, 16, dtype=torch.bfloat16)
    y, *_ = oracle.produce_cast(oracle.PROD_MODULATE, _bits(x), _bits(a), _bits(z), 1.0, oracle.E4M3)
    assert (y == 0).all()
    # overflow of the bf16 range -> +0
    big = torch.full((32, 16), 3.0e38, dtype=torch.bfloat16)
    y, *_ = oracle.produce_cast(oracle.PROD_MODULATE, _bits(big), _bits(big),
                                _bits(torch.full((32, 16), 0.5, dtype=torch.bfloat16)), 1.0, oracle.E4M3)
    assert (y == 0).all()


def test_cast_part_is_the_cast_of_y():
    x, a = _rand_bf16((128, 64), 10), _rand_bf16((128, 64), 11)
    y, q, qt, amax, sinv = oracle.produce_cast(oracle.PROD_ADD, _bits(x), _bits(a), None, 37.0,
                                               oracle.E4M3)
    cq, cqt, camax, csinv = oracle.cast_transpose_amax(y, 37.0, oracle.E4M3)
    np.testing.assert_array_equal(q, cq)
    np.testing.assert_array_equal(qt, cqt)
    assert amax == camax and sinv == csinv


def test_bad_arguments():
    x = np.zeros((4, 4), np.uint16)
    with pytest.raises(ValueError):
        oracle.produce_cast(oracle.PROD_MODULATE, x, x, None, 1.0, oracle.E4M3)   # b missing
    with pytest.raises(ValueError):
        oracle.produce_cast(oracle.PROD_ADD2, x, x, None, 1.0, oracle.E4M3)       # b missing
    with pytest.raises(ValueError):
        oracle.produce_cast(4, x, x, x, 1.0, oracle.E4M3)
