"""Pins of the oracle's modulation gradient (orc_modulate_backward): the
gradient of y = a * x / b, the modulation of the toy block in "CPU Overhead
of te.Linear FP8 Layers" (the block input times one column slice of the
modulation linear's output, divided by another), with respect to x, a and b.

The reference is torch's autograd in float64, which derives the gradient of
the forward expression itself: the oracle's bf16 results must lie within
half a bf16 ulp of it, plus the few fp32 roundings the oracle's steps make
(derived bound below).  Closed forms and the special values pin the rest.
Where the finite modulation replaced a non-finite quotient the oracle's
gradients are +0 (the forward is a constant there); autograd of nan_to_num
masks the upstream gradient instead and then multiplies that 0 by 1/b, so
at a zero divisor it gives NaN: those entries are pinned by definition."""
import numpy as np
import pytest
import torch

import oracle

# |got - exact| <= (1/2 + 2^-14) ulp(exact): at most three fp32 roundings
# before the result (each 2^-24 relative; the bf16 product a*x is exact in
# fp32), i.e. under 2^-14 of a bf16 ulp, then one round-to-nearest-even to
# bf16 (half an ulp).  Truncation would reach a whole ulp.
ULP_BOUND = 0.5 + 2.0 ** -14


def _ulp(w: np.ndarray) -> np.ndarray:
    """bf16 ulp at |w| (8 significant bits), in the binade of w."""
    return np.exp2(np.floor(np.log2(np.abs(w))) - 7)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.bfloat16).contiguous().view(torch.int16).numpy().view(np.uint16)


def _f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _autograd(dy, x, a, b, finite):
    """float64 autograd of y = a*x/b (finite: nan_to_num of it with every
    non-finite value -> 0, whose gradient is zero there)."""
    xs, as_, bs = (torch.tensor(_f64(_bits(t)), requires_grad=True) for t in (x, a, b))
    y = as_ * xs / bs
    if finite:
        y = torch.nan_to_num(y, nan=0.0, posinf=0.0, neginf=0.0)
    y.backward(torch.tensor(_f64(_bits(dy))))
    return xs.grad.numpy(), as_.grad.numpy(), bs.grad.numpy()


def _rand(shape, seed, lo, hi):
    g = torch.Generator().manual_seed(seed)
    mag = torch.exp(torch.empty(shape).uniform_(np.log(lo), np.log(hi), generator=g))
    sign = torch.where(torch.rand(shape, generator=g) < 0.5, -1.0, 1.0)
    return (mag * sign).to(torch.bfloat16)


@pytest.mark.parametrize("op", [oracle.PROD_MODULATE, oracle.PROD_MODULATE_FINITE])
def test_random_values_against_float64_autograd(op):
    shape = (64, 96)
    dy, x = _rand(shape, 1, 1e-3, 1e2), _rand(shape, 2, 1e-2, 1e2)
    a, b = _rand(shape, 3, 1e-2, 1e2), _rand(shape, 4, 1e-2, 1e2)
    got = oracle.modulate_backward(op, _bits(dy), _bits(x), _bits(a), _bits(b))
    want = _autograd(dy, x, a, b, finite=op == oracle.PROD_MODULATE_FINITE)
    for g, w, name in zip(got, want, ("dx", "da", "db")):
        gv = _f64(g)
        assert np.isfinite(w).all() and (w != 0).all()
        err_ulp = np.abs(gv - w) / _ulp(w)
        assert (err_ulp <= ULP_BOUND).all(), (name, float(err_ulp.max()))


def test_rounding_is_to_nearest_not_truncation():
    """Exact quotients that fall between two bf16 values: the oracle must take
    the nearer one (truncation would take the one towards zero)."""
    # dy = 1, b = 3: t = 1/3; dx = t*a with a = 1 -> 0.3333.. rounds up in bf16
    one = torch.ones(1, 1, dtype=torch.bfloat16)
    three = torch.full((1, 1), 3.0, dtype=torch.bfloat16)
    dx, da, db = oracle.modulate_backward(oracle.PROD_MODULATE, _bits(one), _bits(one),
                                          _bits(one), _bits(three))
    exact = 1.0 / 3.0
    lo = float(torch.tensor(exact).to(torch.bfloat16))           # torch rounds to nearest
    assert _f64(dx)[0, 0] == lo == _f64(da)[0, 0]
    assert _f64(db)[0, 0] == float(torch.tensor(-exact / 3.0).to(torch.bfloat16))


def test_closed_forms():
    t = lambda v: torch.full((1, 1), v, dtype=torch.bfloat16)
    dx, da, db = oracle.modulate_backward(oracle.PROD_MODULATE, _bits(t(1.0)), _bits(t(1.0)),
                                          _bits(t(1.0)), _bits(t(1.0)))
    assert (_f64(dx)[0, 0], _f64(da)[0, 0], _f64(db)[0, 0]) == (1.0, 1.0, -1.0)
    # dy = 2, x = 5, a = 3, b = 4: y = 3.75; dx = 2*3/4, da = 2*5/4, db = -2*3.75/4
    dx, da, db = oracle.modulate_backward(oracle.PROD_MODULATE, _bits(t(2.0)), _bits(t(5.0)),
                                          _bits(t(3.0)), _bits(t(4.0)))
    assert (_f64(dx)[0, 0], _f64(da)[0, 0], _f64(db)[0, 0]) == (1.5, 2.5, -1.875)
    # the gradient is linear in dy: dy = 0 gives zeros of the right signs
    dx, da, db = oracle.modulate_backward(oracle.PROD_MODULATE, _bits(t(0.0)), _bits(t(5.0)),
                                          _bits(t(3.0)), _bits(t(4.0)))
    assert (dx[0, 0], da[0, 0], db[0, 0]) == (0x0000, 0x0000, 0x8000)


def test_zero_divisor_page_op_against_float64_autograd():
    """b = +-0 with a*x != 0: the page's modulation is +-inf there, and so is
    every gradient, with autograd's signs."""
    g = torch.Generator().manual_seed(7)
    dy = _rand((8, 16), 5, 0.1, 10.0)
    x, a = _rand((8, 16), 6, 0.1, 10.0), _rand((8, 16), 7, 0.1, 10.0)
    b = torch.where(torch.rand(8, 16, generator=g) < 0.5, 0.0, -0.0).to(torch.bfloat16)
    got = oracle.modulate_backward(oracle.PROD_MODULATE, _bits(dy), _bits(x), _bits(a), _bits(b))
    want = _autograd(dy, x, a, b, finite=False)
    for gb, w in zip(got, want):
        np.testing.assert_array_equal(_f64(gb), w)      # +-inf, same signs


def test_finite_op_zeroes_where_the_forward_was_replaced():
    """Op FINITE: zeros exactly where bf16(a*x/b) is not finite (zero divisors,
    0/0, and a finite fp32 quotient that rounds past the bf16 range), the page
    op's values elsewhere; float64 autograd of nan_to_num agrees."""
    t = lambda vals: torch.tensor([vals], dtype=torch.bfloat16)
    dy = t([1.0, 1.0, 1.0, 2.0, -3.0])
    x = t([1.0, 0.0, 3.0e38, 5.0, 0.5])
    a = t([2.0, 0.0, 2.0, 3.0, 0.25])
    b = t([0.0, 0.0, 1.0, 4.0, -2.0])
    fin = oracle.modulate_backward(oracle.PROD_MODULATE_FINITE, _bits(dy), _bits(x), _bits(a),
                                   _bits(b))
    page = oracle.modulate_backward(oracle.PROD_MODULATE, _bits(dy), _bits(x), _bits(a), _bits(b))
    kept = np.array([False, False, False, True, True])
    for f, p in zip(fin, page):
        assert (f[0, ~kept] == 0).all()
        np.testing.assert_array_equal(f[0, kept], p[0, kept])
    # where the forward is finite, float64 autograd of nan_to_num agrees
    want = _autograd(dy, x, a, b, finite=True)
    for f, w in zip(fin, want):
        np.testing.assert_array_equal(_f64(f)[0, [3, 4]], w[0, [3, 4]])


def test_strided_inputs_and_bad_arguments():
    rng = np.random.default_rng(3)
    wide = (rng.integers(0x3C00, 0x4100, size=(16, 40))).astype(np.uint16)
    dy, x, a, b = wide[:, 0:8], wide[:, 8:16], wide[:, 16:24], wide[:, 24:32]
    got = oracle.modulate_backward(oracle.PROD_MODULATE, dy, x, a, b)
    ref = oracle.modulate_backward(oracle.PROD_MODULATE, *(np.ascontiguousarray(t)
                                                           for t in (dy, x, a, b)))
    for g, r in zip(got, ref):
        np.testing.assert_array_equal(g, r)
    with pytest.raises(ValueError):
        oracle.modulate_backward(oracle.PROD_ADD, dy, x, a, b)
