"""GPU parity of the producer-fused cast (fp8_produce_cast_transpose_amax):
the toy block's elementwise producers rounded to bf16 and the cast of the
result, bit-exact against the oracle (y, codes, transpose, amax,
scale-inverse), through the C ABI."""
import numpy as np
import pytest
import torch

import delayed_scaling_linear_amd as dsl
import oracle
from tests.gpu_util import DEV, bf16_values, bits8, bits16, f32_bits

pytestmark = pytest.mark.gpu


def _bits_view(t: torch.Tensor) -> np.ndarray:
    """bf16 bits of a (possibly strided) CPU tensor as a numpy view with the same strides."""
    base = t.contiguous() if t.storage_offset() == 0 and t.is_contiguous() else None
    if base is not None:
        return base.view(torch.int16).numpy().view(np.uint16)
    full = t._base if t._base is not None else t
    fb = full.view(torch.int16).numpy().view(np.uint16)
    r0, c0 = divmod(t.storage_offset(), full.stride(0))
    return fb[r0:r0 + t.shape[0], c0:c0 + t.shape[1]]


def _run_and_check(op, x, a, b, scale, fmt, q=True, qt=True):
    """x, a, b: CPU bf16 tensors (b may be None); views of wider tensors allowed."""
    rows, cols = x.shape
    # move the underlying storage once so device views keep the host strides
    def to_dev(t):
        if t is None:
            return None
        if t._base is not None:
            full = t._base.to(DEV)
            r0, c0 = divmod(t.storage_offset(), t._base.stride(0))
            return full[r0:r0 + t.shape[0], c0:c0 + t.shape[1]]
        return t.to(DEV)
    xd, ad, bd = to_dev(x), to_dev(a), to_dev(b)
    y = torch.full((rows, cols), -7.0, dtype=torch.bfloat16, device=DEV)
    out = dsl.Float8Tensor.empty(rows, cols, fmt, data=q, transpose=qt, device=DEV)
    s = torch.tensor([scale], dtype=torch.float32, device=DEV)
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    dsl.fp8_produce_cast_transpose_amax(op, xd, ad, bd, y, s, out, amax)
    torch.cuda.synchronize()
    oy, oq, oqt, oamax, osinv = oracle.produce_cast(
        op, _bits_view(x), _bits_view(a), None if b is None else _bits_view(b), scale, fmt,
        want_q=q, want_qt=qt)
    np.testing.assert_array_equal(bits16(y), oy)
    if q:
        np.testing.assert_array_equal(bits8(out.data), oq)
    if qt:
        np.testing.assert_array_equal(bits8(out.data_t), oqt)
    assert f32_bits(amax)[0] == np.float32(oamax).view(np.uint32)
    assert f32_bits(out.scale_inv)[0] == np.float32(osinv).view(np.uint32)
    return y


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("extra", [16, 48, 64, 80, 112])
@pytest.mark.parametrize("op", [oracle.PROD_MODULATE, oracle.PROD_ADD2])
def test_every_column_residue_of_a_tile(extra, op):
    """Right-edge tiles of every residue width: each 8-column chunk is
    produced and written as y only when it lies inside the tensor."""
    shape = (48, 128 + extra)
    x, a = _rand(shape, 3000 + extra), _rand(shape, 3100 + extra, 0.5)
    b = _rand(shape, 3200 + extra, 2.0)
    _run_and_check(op, x, a, b, 9.0, oracle.E4M3)


@pytest.mark.parametrize("shape", [(16, 16), (400, 272), (272, 400), (1024, 2048)])
@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_modulate_shapes(shape, fmt):
    x, a, b = _rand(shape, 1), _rand(shape, 2), _rand(shape, 3, 0.7)
    _run_and_check(oracle.PROD_MODULATE, x, a, b, 41.0, fmt)


@pytest.mark.parametrize("shape", [(16, 16), (400, 272), (1024, 2048)])
@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_add_shapes(shape, fmt):
    x, a = _rand(shape, 4), _rand(shape, 5, 3.0)
    _run_and_check(oracle.PROD_ADD, x, a, None, 41.0, fmt)


@pytest.mark.parametrize("shape", [(16, 16), (400, 272), (1024, 2048)])
@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_add2_shapes(shape, fmt):
    x, a, b = _rand(shape, 16), _rand(shape, 17, 3.0), _rand(shape, 18, 0.05)
    _run_and_check(oracle.PROD_ADD2, x, a, b, 41.0, fmt)


def test_add2_rounds_after_each_term():
    """1 + 2^-8 + 2^-8: each sum is a tie that rounds back to 1."""
    one = torch.ones(32, 32, dtype=torch.bfloat16)
    e = torch.full((32, 32), 2.0 ** -8, dtype=torch.bfloat16)
    y = _run_and_check(oracle.PROD_ADD2, one, e, e, 1.0, oracle.E4M3)
    assert (bits16(y) == 0x3F80).all()


def test_toy_block_shapes_with_column_slices():
    """shift, scale = columns [0, 2048) and [2048, 4096) of the modulation
    output [8192, 12288]; the qkv residual = columns [0, 2048) of [8192, 6144]."""
    mod = _rand((8192, 12288), 6, 0.5)
    x = (torch.rand(8192, 2048, generator=torch.Generator().manual_seed(7))).to(torch.bfloat16)
    y = _run_and_check(oracle.PROD_MODULATE, x, mod[:, :2048], mod[:, 2048:4096], 3.5, oracle.E4M3)
    qkv = _rand((8192, 6144), 8, 0.02)
    _run_and_check(oracle.PROD_ADD, y.cpu(), qkv[:, :2048], None, 3.5, oracle.E4M3, qt=False)
    # x + attn_q [8192, 2048] + attn_k[:, :2048] of [8192, 4096]
    q_out = _rand((8192, 2048), 19, 0.02)
    k_out = _rand((8192, 4096), 20, 0.02)
    _run_and_check(oracle.PROD_ADD2, y.cpu(), q_out, k_out[:, :2048], 3.5, oracle.E4M3)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_special_values(fmt):
    x, a, b = _rand((64, 64), 9), _rand((64, 64), 10), _rand((64, 64), 11)
    b[0, :] = 0.0                        # a*x/0 -> +-inf -> the cast saturates
    b[5, :] = -0.0                       # the zero's sign flips the infinity
    x[1, :] = 0.0
    b[1, :] = 0.0                        # 0/0 -> NaN (0x7FC0) -> code 0x7F
    x[2, :] = 3.0e38
    a[2, :] = 3.0e38                     # fp32 product overflows -> inf
    x[3, :], a[3, :], b[3, :] = 1.0e20, 1.0e20, 1.0e-5   # beyond bf16 only -> inf
    x[4, :], b[4, :] = float("inf"), float("inf")        # inf/inf -> NaN
    y = _run_and_check(oracle.PROD_MODULATE, x, a, b, 1.0, fmt)
    v = bits16(y)
    assert np.isin(v[[0, 2, 3, 5]], [0x7F80, 0xFF80]).all()
    assert (v[1] == 0x7FC0).all() and (v[4] == 0x7FC0).all()
    x2, a2 = _rand((64, 64), 12), _rand((64, 64), 13)
    x2[0, 0], a2[1, 1] = float("nan"), float("inf")
    x2[2, 2], a2[2, 2] = float("-inf"), float("inf")
    y = _run_and_check(oracle.PROD_ADD, x2, a2, None, 1.0, oracle.E5M2)
    v = bits16(y)
    assert v[0, 0] == 0x7FC0 and v[2, 2] == 0x7FC0 and v[1, 1] == 0x7F80
    b2 = _rand((64, 64), 21)
    b2[3, 3], a2[3, 3] = float("-inf"), float("inf")    # NaN at the second add
    b2[4, 4] = float("nan")
    y = _run_and_check(oracle.PROD_ADD2, x2, a2, b2, 1.0, oracle.E4M3)
    v = bits16(y)
    assert v[0, 0] == 0x7FC0 and v[3, 3] == 0x7FC0 and v[4, 4] == 0x7FC0


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_finite_modulation(fmt):
    """The library's finite modulation: the page's quotient with non-finite
    results replaced by +0, on special values and a ragged shape."""
    x, a, b = _rand((400, 272), 25), _rand((400, 272), 26), _rand((400, 272), 27, 0.7)
    b[0, :] = 0.0
    x[1, :] = 0.0
    b[1, :] = 0.0
    x[2, :], a[2, :], b[2, :] = 1.0e20, 1.0e20, 1.0e-5
    a[3, :] = float("nan")
    y = _run_and_check(oracle.PROD_MODULATE_FINITE, x, a, b, 41.0, fmt)
    v = bits16(y)
    assert (v[:4] == 0).all() and np.isfinite(bf16_values(v)).all()


def test_toy_block_modulation_with_zero_divisors():
    """The modulation at the block's real shape with a few exact zeros in the
    divisor slice (a bf16 linear output can round to zero): the infinities
    and NaNs flow into the cast, and the amax becomes NaN, as in the oracle."""
    mod = _rand((8192, 12288), 22, 0.5)
    g = torch.Generator().manual_seed(23)
    zr = torch.randint(0, 8192, (64,), generator=g)
    zc = torch.randint(2048, 4096, (64,), generator=g)
    mod[zr, zc] = 0.0
    x = torch.rand(8192, 2048, generator=torch.Generator().manual_seed(24)).to(torch.bfloat16)
    x[zr[:8], zc[:8] - 2048] = 0.0                      # 0/0 at eight of them
    y = _run_and_check(oracle.PROD_MODULATE, x, mod[:, :2048], mod[:, 2048:4096], 3.5,
                       oracle.E4M3)
    assert np.isnan(bf16_values(bits16(y))).any()


def test_noop_flag_writes_nothing():
    x, a = _rand((64, 64), 14).to(DEV), _rand((64, 64), 15).to(DEV)
    y = torch.full((64, 64), -7.0, dtype=torch.bfloat16, device=DEV)
    out = dsl.Float8Tensor.empty(64, 64, 0, device=DEV)
    out.data.fill_(0xAA)
    flag = torch.ones(1, dtype=torch.int32, device=DEV)
    amax = torch.zeros(1, device=DEV)
    dsl.fp8_produce_cast_transpose_amax(dsl.PRODUCE_ADD, x, a, None, y,
                                        torch.ones(1, device=DEV), out, amax, noop_flag=flag)
    torch.cuda.synchronize()
    assert (y.float() == -7.0).all() and (out.data == 0xAA).all() and float(amax[0]) == 0.0


def _grad_check(op, dy, x, a, b, outs=None):
    """fp8_produce_modulate_backward on device copies of the CPU bf16 tensors
    (views of wider tensors keep their strides), bit-exact against the oracle."""
    def to_dev(t):
        if t._base is not None:
            full = t._base.to(DEV)
            r0, c0 = divmod(t.storage_offset(), t._base.stride(0))
            return full[r0:r0 + t.shape[0], c0:c0 + t.shape[1]]
        return t.to(DEV)
    if outs is None:
        outs = [torch.full(dy.shape, -3.0, dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    dsl.fp8_produce_modulate_backward(op, to_dev(dy), to_dev(x), to_dev(a), to_dev(b), *outs)
    torch.cuda.synchronize()
    want = oracle.modulate_backward(op, _bits_view(dy), _bits_view(x), _bits_view(a), _bits_view(b))
    for got, w, name in zip(outs, want, ("dx", "da", "db")):
        np.testing.assert_array_equal(bits16(got), w, err_msg=name)
    return outs


@pytest.mark.parametrize("shape", [(16, 8), (272, 400), (1000, 2056)])
@pytest.mark.parametrize("op", [oracle.PROD_MODULATE, oracle.PROD_MODULATE_FINITE])
def test_modulate_backward_shapes(shape, op):
    dy, x = _rand(shape, 11), _rand(shape, 12, 3.0)
    a, b = _rand(shape, 13, 0.5), _rand(shape, 14, 0.8)
    _grad_check(op, dy, x, a, b)


@pytest.mark.parametrize("op", [oracle.PROD_MODULATE, oracle.PROD_MODULATE_FINITE])
def test_modulate_backward_at_the_block_layout(op):
    """The toy block's shapes: the gain and divisor are column slices of the
    modulation linear's [8192, 12288] output, and da, db go straight into
    the first two column slices of its [8192, 12288] output gradient."""
    M, H = 8192, 2048
    m = _rand((M, 6 * H), 21, 0.7)
    dy, h0 = _rand((M, H), 22, 1e-3), _rand((M, H), 23)
    gain, div = m[:, :H], m[:, H:2 * H]
    dmod = torch.zeros(M, 6 * H, dtype=torch.bfloat16, device=DEV)
    dh0 = torch.empty(M, H, dtype=torch.bfloat16, device=DEV)
    _grad_check(op, dy, h0, gain, div, outs=[dh0, dmod[:, :H], dmod[:, H:2 * H]])
    assert int(torch.count_nonzero(dmod[:, 2 * H:])) == 0       # untouched columns


@pytest.mark.parametrize("op", [oracle.PROD_MODULATE, oracle.PROD_MODULATE_FINITE])
def test_modulate_backward_specials(op):
    """Zero divisors of both signs, 0/0, infinite and NaN operands, and a
    quotient that overflows bf16: the finite op zeroes exactly where the
    forward wrote its constant."""
    inf, nan = float("inf"), float("nan")
    vals_x = [1.0, 0.0, 3.0e38, 2.0, inf, nan, 1.0, -0.0, 1e-30, 5.0, 1.0, 2.0, 7.0, 0.5, -1.0, 3.0]
    vals_a = [2.0, 0.0, 2.0, inf, 1.0, 1.0, nan, 1.0, 1e-30, 3.0, 1.0, 0.0, 1.0, 1.0, 1.0, 1.0]
    vals_b = [0.0, 0.0, 1.0, 1.0, 2.0, 1.0, 1.0, -0.0, 1e-30, 4.0, inf, 1.0, 0.0, -0.0, 1.0, nan]
    vals_g = [1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 2.0, 1.0, inf, -1.0, 1.0, nan, 1.0]
    t = lambda v: torch.tensor([v], dtype=torch.bfloat16)
    _grad_check(op, t(vals_g), t(vals_x), t(vals_a), t(vals_b))
