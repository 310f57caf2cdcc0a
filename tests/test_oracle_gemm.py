"""Pins for the oracle's per-tensor-scaled FP8 product (CPU only).

The definition is torch._scaled_mm's (Part 2 blog): the first operand
row-major, the second transposed, per-tensor scales, optional bf16 bias.  Pins:
K = 1 outer products (exact), an FP8 identity operand, all-ones operands
(acc = K exactly), exact integer / rational brute force at the blog's 16x16x16
demo shape and at the tiny forward shape (128 x 512 x 256), and the
forward / dgrad / wgrad compositions against numpy products of the decoded,
untransposed matrices.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import exact


def _codes(rng, shape, fmt, lo_exp=-6, hi_exp=6):
    """Random finite FP8 codes (NaN and inf codes excluded)."""
    t = oracle.decode_table(fmt)
    ok = [c for c in range(256) if np.isfinite(t[c]) and 2.0 ** lo_exp <= abs(t[c]) <= 2.0 ** hi_exp
          or t[c] == 0]
    return rng.choice(np.array(ok, dtype=np.uint8), size=shape)


def _bf16_bits(vals):
    import torch
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _exact_int_products(A, fa, B, fb):
    """Exact A.B^T of decoded operands as (integer matrix, power-of-two scale)."""
    sa = 9 if fa == oracle.E4M3 else 16     # 2^-9 / 2^-16: smallest subnormals
    sb = 9 if fb == oracle.E4M3 else 16
    ia = (oracle.fp8_decode(A, fa) * 2.0 ** sa).astype(np.int64)
    ib = (oracle.fp8_decode(B, fb) * 2.0 ** sb).astype(np.int64)
    assert (ia.astype(np.float64) == oracle.fp8_decode(A, fa) * 2.0 ** sa).all()
    bound = int(np.abs(ia).max(initial=0)) * int(np.abs(ib).max(initial=0)) * A.shape[1]
    assert bound < 2 ** 62, "integer brute force would overflow"
    return ia @ ib.T, Fraction(1, 2 ** (sa + sb))


def _exact_out(acc_int, unit, sinv_a, sinv_b, bias, out_kind):
    M, N = acc_int.shape
    sa, sb = exact.f32_fraction(sinv_a), exact.f32_fraction(sinv_b)
    out = np.empty((M, N), np.uint16 if out_kind == oracle.OUT_BF16 else np.float32)
    bvals = None if bias is None else [Fraction(float(v)) for v in oracle.bf16_bits_to_f32(bias)]
    for i in range(M):
        for j in range(N):
            y = Fraction(int(acc_int[i, j])) * unit * sa * sb
            if bvals is not None:
                y += bvals[j]
            out[i, j] = exact.to_bf16_bits(y) if out_kind == oracle.OUT_BF16 else exact.to_f32(y)
    return out


def test_outer_product_k1_is_exact():
    rng = np.random.default_rng(1)
    A = _codes(rng, (9, 1), oracle.E4M3)
    B = _codes(rng, (13, 1), oracle.E5M2)
    y = oracle.gemm_nt(A, oracle.E4M3, B, oracle.E5M2, 1.0, 1.0)
    prod = np.outer(oracle.fp8_decode(A[:, 0], 0), oracle.fp8_decode(B[:, 0], 1))
    # Products of FP8 significands have at most 4 + 3 bits: exact in bf16.
    want = (prod.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(y, want)


def test_identity_operand():
    rng = np.random.default_rng(2)
    M, K = 24, 32
    A = _codes(rng, (M, K), oracle.E4M3)
    eye = np.zeros((K, K), np.uint8)
    np.fill_diagonal(eye, 0x38)                      # 1.0 in E4M3
    assert oracle.fp8_decode(np.uint8(0x38), 0) == 1.0
    y = oracle.gemm_nt(A, oracle.E4M3, eye, oracle.E4M3, 0.25, 2.0, out_kind=oracle.OUT_FP32)
    np.testing.assert_array_equal(y, (oracle.fp8_decode(A, 0) * 0.5).astype(np.float32))


def test_all_ones_accumulates_k():
    K = 4096
    A = np.full((3, K), 0x38, np.uint8)
    B = np.full((5, K), 0x3C, np.uint8)              # 1.0 in E5M2
    assert oracle.fp8_decode(np.uint8(0x3C), 1) == 1.0
    y = oracle.gemm_nt(A, oracle.E4M3, B, oracle.E5M2, 1.0, 1.0, out_kind=oracle.OUT_FP32)
    assert (y == K).all()


@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_scaled_mm_demo_shape_exact(fa, fb):
    """16x16x16 with bias and power-of-two scale-inverses: bit-exact."""
    rng = np.random.default_rng(10 + 2 * fa + fb)
    A = _codes(rng, (16, 16), fa)
    B = _codes(rng, (16, 16), fb)
    bias = _bf16_bits(rng.standard_normal(16).astype(np.float32))
    acc, unit = _exact_int_products(A, fa, B, fb)
    for kind in (oracle.OUT_BF16, oracle.OUT_FP32):
        y = oracle.gemm_nt(A, fa, B, fb, 0.125, 4.0, bias=bias, out_kind=kind)
        np.testing.assert_array_equal(y, _exact_out(acc, unit, 0.125, 4.0, bias, kind))


def test_tiny_forward_shape_exact():
    """128 x 512 x 256 (the tiny forward layer), non-square so a transposed
    operand or swapped index cannot pass; general fp32 scale-inverses."""
    rng = np.random.default_rng(20)
    M, N, K = 128, 512, 256
    A = _codes(rng, (M, K), 0)
    B = _codes(rng, (N, K), 0, lo_exp=-9, hi_exp=-2)
    bias = _bf16_bits((rng.standard_normal(N) * 0.02).astype(np.float32))
    sa, sb = np.float32(1 / 3.7), np.float32(1 / 448.0 * 1.3)
    y = oracle.gemm_nt(A, 0, B, 0, float(sa), float(sb), bias=bias)
    acc, unit = _exact_int_products(A, 0, B, 0)
    want = _exact_out(acc, unit, sa, sb, bias, oracle.OUT_BF16)
    # The oracle's epilogue is fp64 (2^-53 relative): it can only differ from
    # the exactly rounded bf16 when the exact value sits within 2^-50 of a bf16
    # rounding boundary.  Require bit equality everywhere else.
    diff = y != want
    if diff.any():
        yf = oracle.bf16_bits_to_f32(y[diff]).astype(np.float64)
        wf = oracle.bf16_bits_to_f32(want[diff]).astype(np.float64)
        assert np.all(np.abs(yf - wf) <= np.abs(wf) * 2.0 ** -7)
        assert diff.sum() <= 2
    sampled_rows = rng.integers(0, M, 300)
    sampled_cols = rng.integers(0, N, 300)
    ys = oracle.gemm_nt_sampled(A, 0, B, 0, float(sa), float(sb), sampled_rows, sampled_cols,
                                bias=bias)
    np.testing.assert_array_equal(ys, y[sampled_rows, sampled_cols])


def test_linear_passes_compose_to_plain_products():
    """fwd Y = X W^T, dgrad dX = dY W (via W's transpose), wgrad dW = dY^T X
    (via both transposes), against numpy products of the untransposed decoded
    matrices."""
    rng = np.random.default_rng(30)
    M, N, K = 40, 24, 56
    X = _codes(rng, (M, K), 0)
    W = _codes(rng, (N, K), 0)
    dY = _codes(rng, (M, N), 1, lo_exp=-10, hi_exp=-2)
    dx, dw, dy = (oracle.fp8_decode(a, f) for a, f in ((X, 0), (W, 0), (dY, 1)))
    f32 = oracle.OUT_FP32
    y = oracle.gemm_nt(X, 0, W, 0, 1.0, 1.0, out_kind=f32)
    np.testing.assert_allclose(y, dx @ dw.T, rtol=1e-6)
    dX = oracle.gemm_nt(dY, 1, np.ascontiguousarray(W.T), 0, 1.0, 1.0, out_kind=f32)
    np.testing.assert_allclose(dX, dy @ dw, rtol=1e-6)
    dW = oracle.gemm_nt(np.ascontiguousarray(dY.T), 1, np.ascontiguousarray(X.T), 0, 1.0, 1.0,
                        out_kind=f32)
    np.testing.assert_allclose(dW, dy.T @ dx, rtol=1e-6)


def test_nan_code_propagates():
    A = np.full((2, 4), 0x38, np.uint8)
    A[1, 2] = 0x7F
    B = np.full((3, 4), 0x38, np.uint8)
    y = oracle.gemm_nt(A, 0, B, 0, 1.0, 1.0, out_kind=oracle.OUT_FP32)
    assert (y[0] == 4).all() and np.isnan(y[1]).all()
