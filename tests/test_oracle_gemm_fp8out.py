"""Pins for the oracle's FP8-output product (CPU only).

torch._scaled_mm with an FP8 out_dtype returns the FP8 output and its amax
(Part 2 blog, the torch._scaled_mm example).  The oracle reads this as the
fp32 product followed by the cast with the output's scale; the amax is that of
the unscaled product.  Pins, each by a route that shares nothing with the
oracle's code:
  * exact rational products (integer brute force) rounded to fp32, scaled by
    one fp32 multiply in numpy, clamped, and cast by torch's own float8
    conversion, at the blog's 16x16x16 demo shape, every operand and output
    format, with bias and a non-power-of-two output scale;
  * closed forms: all-ones operands saturate (E4M3) or hit an exact code
    (E5M2) with amax = K; an FP8 identity operand with sinv_a * sinv_b *
    scale = 1 reproduces the operand's own codes;
  * a NaN code in an operand row makes that output row NaN codes and the
    amax NaN, leaving the other rows alone.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import exact

TORCH_DT = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}
FMAX = {oracle.E4M3: 448.0, oracle.E5M2: 57344.0}


def _codes(rng, shape, fmt, lo_exp=-6, hi_exp=6):
    """Random finite FP8 codes with magnitudes in [2^lo_exp, 2^hi_exp] or 0,
    picked from the torch decode of every byte (not the oracle's)."""
    vals = torch.arange(256, dtype=torch.uint8).view(TORCH_DT[fmt]).float().numpy()
    ok = [c for c in range(256) if np.isfinite(vals[c]) and
          (vals[c] == 0 or 2.0 ** lo_exp <= abs(vals[c]) <= 2.0 ** hi_exp)]
    return rng.choice(np.array(ok, dtype=np.uint8), size=shape), vals


def _torch_cast(v32: np.ndarray, fmt: int) -> np.ndarray:
    """Saturating cast through torch: clamp to the format's range (torch's
    own conversion does not saturate), then torch's round-to-nearest-even."""
    c = np.clip(v32, -FMAX[fmt], FMAX[fmt]).astype(np.float32)
    return torch.from_numpy(c).to(TORCH_DT[fmt]).view(torch.uint8).numpy()


@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("fo", [oracle.E4M3, oracle.E5M2])
def test_demo_shape_against_exact_products_and_torch_cast(fa, fb, fo):
    rng = np.random.default_rng(100 + 4 * fa + 2 * fb + fo)
    A, ta = _codes(rng, (16, 16), fa)
    B, tb = _codes(rng, (16, 16), fb)
    bias_f = (rng.standard_normal(16) * 4).astype(np.float32)
    bias = (torch.from_numpy(bias_f).to(torch.bfloat16).view(torch.int16).numpy()
            .view(np.uint16))
    sa, sb = np.float32(1 / 3.0), np.float32(0.75)
    scale = np.float32(0.7) if fo == oracle.E4M3 else np.float32(91.3)
    # exact v, rounded once to fp32
    fa_ = [[Fraction(float(ta[c])) for c in row] for row in A]
    fb_ = [[Fraction(float(tb[c])) for c in row] for row in B]
    bvals = torch.from_numpy(bias.view(np.int16)).view(torch.bfloat16).float().numpy()
    v = np.empty((16, 16), np.float32)
    for i in range(16):
        for j in range(16):
            acc = sum(x * y for x, y in zip(fa_[i], fb_[j]))
            v[i, j] = exact.to_f32(acc * exact.f32_fraction(sa) * exact.f32_fraction(sb)
                                   + Fraction(float(bvals[j])))
    want = _torch_cast(v * scale, fo)             # one fp32 multiply per element
    codes, vo, amax, sinv = oracle.gemm_nt_fp8out(A, fa, B, fb, float(sa), float(sb),
                                                  float(scale), fo, bias=bias)
    np.testing.assert_array_equal(vo, v)
    np.testing.assert_array_equal(codes, want)
    assert amax == np.abs(v).max()
    assert sinv == np.float32(1.0) / scale


def test_all_ones_saturates_or_is_exact():
    K = 2048
    A = np.full((3, K), 0x38, np.uint8)              # 1.0 in E4M3
    B = np.full((5, K), 0x38, np.uint8)
    c4, _, amax, _ = oracle.gemm_nt_fp8out(A, 0, B, 0, 1.0, 1.0, 1.0, oracle.E4M3)
    assert (c4 == 0x7E).all() and amax == K          # 2048 > 448: saturates
    c5, _, amax, _ = oracle.gemm_nt_fp8out(A, 0, B, 0, 1.0, 1.0, 1.0, oracle.E5M2)
    # 2048 = 2^11: E5M2 exponent field 11 + 15 = 26, mantissa 0
    assert (c5 == (26 << 2)).all() and amax == K
    An = np.full((3, K), 0xB8, np.uint8)             # -1.0 in E4M3
    cn, _, amax, _ = oracle.gemm_nt_fp8out(An, 0, B, 0, 1.0, 1.0, 1.0, oracle.E4M3)
    assert (cn == 0xFE).all() and amax == K


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_identity_operand_reproduces_codes(fmt):
    rng = np.random.default_rng(7 + fmt)
    M, K = 40, 48
    A, vals = _codes(rng, (M, K), fmt, lo_exp=-4, hi_exp=4)
    one = 0x38 if fmt == oracle.E4M3 else 0x3C
    eye = np.zeros((K, K), np.uint8)
    np.fill_diagonal(eye, one)
    # sinv_a * sinv_b * scale = 0.5 * 0.5 * 4 = 1, all powers of two
    codes, v, amax, _ = oracle.gemm_nt_fp8out(A, fmt, eye, fmt, 0.5, 0.5, 4.0, fmt)
    zero = vals[A] == 0                              # +0 and -0 both give +0 sums
    np.testing.assert_array_equal(codes[~zero], A[~zero])
    assert (codes[zero] == 0).all()
    assert amax == np.float32(np.abs(vals[A]).max() * 0.25)


def test_nan_row_propagates_and_dominates_amax():
    rng = np.random.default_rng(3)
    A, _ = _codes(rng, (8, 32), 0)
    B, _ = _codes(rng, (16, 32), 0)
    A[5, 9] = 0x7F                                   # NaN in E4M3
    codes, v, amax, _ = oracle.gemm_nt_fp8out(A, 0, B, 0, 1.0, 1.0, 0.5, oracle.E4M3)
    assert np.isnan(v[5]).all() and np.isfinite(np.delete(v, 5, axis=0)).all()
    assert ((codes[5] & 0x7F) == 0x7F).all()
    assert ((np.delete(codes, 5, axis=0) & 0x7F) != 0x7F).all()
    assert np.isnan(amax)


def test_amax_folds_into_previous_value():
    A = np.full((2, 16), 0x38, np.uint8)
    B = np.full((2, 16), 0x38, np.uint8)
    _, _, amax, _ = oracle.gemm_nt_fp8out(A, 0, B, 0, 1.0, 1.0, 1.0, 0, amax_in=100.0)
    assert amax == 100.0
    _, _, amax, _ = oracle.gemm_nt_fp8out(A, 0, B, 0, 1.0, 1.0, 1.0, 0, amax_in=3.0)
    assert amax == 16.0
