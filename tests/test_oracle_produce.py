"""Pins of the oracle's producer-fused cast: the toy block's elementwise
producers of "CPU Overhead of te.Linear FP8 Layers" (TEBlock.forward: the
modulation, a product divided by a quotient of linear outputs, and the
residual adds), rounded to bf16.  Checked against torch's own CPU bf16
arithmetic (an independent implementation of the same operations) including
zero divisors, 0/0 and overflow, closed forms, and the already pinned cast
oracle.  Nothing is sanitised: infinities and NaNs flow into the cast."""
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
    """torch CPU: fp32 multiply, fp32 division, one rounding to bf16."""
    return (a.float() * x.float() / b.float()).to(torch.bfloat16)


def _assert_same_bf16(y, want):
    """Bit-equal wherever torch's result is a number; NaN exactly where torch
    has NaN (torch's NaN bit pattern depends on its code path, the oracle
    always writes 0x7FC0)."""
    nan = torch.isnan(want).numpy()
    np.testing.assert_array_equal(y[~nan], _bits(want)[~nan])
    assert (y[nan] == 0x7FC0).all()
    return nan


def test_modulate_against_torch():
    a, x, b = _rand_bf16((96, 80), 1), _rand_bf16((96, 80), 2), _rand_bf16((96, 80), 3, 0.5)
    y, *_ = oracle.produce_cast(oracle.PROD_MODULATE, _bits(x), _bits(a), _bits(b), 1.0, oracle.E4M3)
    np.testing.assert_array_equal(y, _bits(_torch_modulate(a, x, b)))


def test_modulate_against_torch_with_zero_divisors_and_overflow():
    """Zero divisors of both signs, 0/0, inf/inf, products that overflow fp32
    and quotients that overflow only the bf16 range: exactly torch's bits."""
    a, x, b = _rand_bf16((64, 64), 31), _rand_bf16((64, 64), 32), _rand_bf16((64, 64), 33, 0.5)
    b[0, :] = 0.0                                  # +-inf by sign of a*x
    b[1, :] = -0.0                                 # the sign of zero flips the infinity
    x[2, :] = 0.0
    b[2, :] = 0.0                                  # 0/0 = NaN
    x[3, :], a[3, :] = 3.0e38, 3.0e38              # fp32 product overflows -> inf
    x[4, :], a[4, :], b[4, :] = 1.0e20, 1.0e20, 1.0e-5   # fp32-finite, beyond bf16 -> inf
    x[5, :], b[5, :] = float("inf"), float("inf")  # inf/inf = NaN
    a[6, :] = float("nan")
    b[7, :] = 1.0e-38                              # large but finite quotients
    y, *_ = oracle.produce_cast(oracle.PROD_MODULATE, _bits(x), _bits(a), _bits(b), 1.0, oracle.E4M3)
    want = _torch_modulate(a, x, b)
    nan = _assert_same_bf16(y, want)
    assert nan[2].all() and nan[5].all() and nan[6].all()
    assert np.isin(y[0:2], [0x7F80, 0xFF80]).all() and np.isin(y[3:5], [0x7F80, 0xFF80]).all()
    ax = (a.float() * x.float()).numpy()
    # division by -0 gives the infinity of the opposite sign
    np.testing.assert_array_equal(y[1] == 0xFF80, ax[1] > 0)


def test_finite_modulation_against_torch_nan_to_num():
    """The library's finite modulation (not on the pages): the page's
    quotient, then every non-finite bf16 result replaced by +0 -- torch's
    nan_to_num(..., nan=0, posinf=0, neginf=0) of the same quotient.  Finite
    results are the page's modulation bit for bit."""
    a, x, b = _rand_bf16((64, 64), 41), _rand_bf16((64, 64), 42), _rand_bf16((64, 64), 43, 0.5)
    b[0, :] = 0.0
    b[1, :] = -0.0
    x[2, :] = 0.0
    b[2, :] = 0.0
    x[3, :], a[3, :], b[3, :] = 1.0e20, 1.0e20, 1.0e-5
    a[4, :] = float("nan")
    y, q, qt, amax, _ = oracle.produce_cast(oracle.PROD_MODULATE_FINITE, _bits(x), _bits(a),
                                            _bits(b), 1.0, oracle.E4M3)
    q_page = _torch_modulate(a, x, b)
    want = torch.nan_to_num(q_page, nan=0.0, posinf=0.0, neginf=0.0)
    np.testing.assert_array_equal(y, _bits(want))
    assert (y[:5] == 0).all()
    yp, *_ = oracle.produce_cast(oracle.PROD_MODULATE, _bits(x), _bits(a), _bits(b), 1.0,
                                 oracle.E4M3)
    fin = torch.isfinite(q_page).numpy()
    np.testing.assert_array_equal(y[fin], yp[fin])
    assert np.isfinite(amax)


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
    _assert_same_bf16(y, _torch_modulate(shift, x, scale))
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
    # a*x/0 is an infinity with the sign of a*x (and of the zero); 0/0 is NaN
    z = torch.zeros(32, 16, dtype=torch.bfloat16)
    y, *_ = oracle.produce_cast(oracle.PROD_MODULATE, _bits(x), _bits(a), _bits(z), 1.0, oracle.E4M3)
    ax = (a.float() * x.float()).numpy()
    np.testing.assert_array_equal(y[ax > 0], 0x7F80)
    np.testing.assert_array_equal(y[ax < 0], 0xFF80)
    np.testing.assert_array_equal(y[ax == 0], 0x7FC0)
    # a quotient beyond the bf16 range rounds to infinity
    big = torch.full((32, 16), 3.0e38, dtype=torch.bfloat16)
    y, *_ = oracle.produce_cast(oracle.PROD_MODULATE, _bits(big), _bits(big),
                                _bits(torch.full((32, 16), 0.5, dtype=torch.bfloat16)), 1.0, oracle.E4M3)
    assert (y == 0x7F80).all()


def test_modulate_specials_reach_the_cast_by_its_rules():
    """The cast part sees the unsanitised y: +-inf saturates to +-max, NaN is
    coded 0x7F with its sign, and the amax records the NaN (it dominates)."""
    one = torch.ones(16, 16, dtype=torch.bfloat16)
    b = torch.ones(16, 16, dtype=torch.bfloat16)
    b[0, :] = 0.0                                        # +inf
    a = one.clone()
    a[1, :] = -1.0
    b[1, :] = 0.0                                        # -inf
    x = one.clone()
    x[2, :] = 0.0
    b[2, :] = 0.0                                        # NaN
    for fmt, maxc in ((oracle.E4M3, 0x7E), (oracle.E5M2, 0x7B)):
        y, q, qt, amax, _ = oracle.produce_cast(oracle.PROD_MODULATE, _bits(x), _bits(a), _bits(b),
                                                2.0, fmt)
        assert (q[0] == maxc).all() and (q[1] == 0x80 | maxc).all() and (q[2] == 0x7F).all()
        np.testing.assert_array_equal(qt, q.T)
        assert np.isnan(amax)


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
        oracle.produce_cast(oracle.PROD_MODULATE_FINITE, x, x, None, 1.0, oracle.E4M3)
    with pytest.raises(ValueError):
        oracle.produce_cast(5, x, x, x, 1.0, oracle.E4M3)
