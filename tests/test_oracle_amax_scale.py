"""Pins for the oracle's amax, transpose and delayed-scaling update (CPU only).

Amax is pinned by brute force against numpy's max(abs) and by constructed
NaN/inf/-0 cases; the transpose against numpy's transpose; the scale update
by closed forms, exact rational rounding and the history-window length of the
DelayedScaling recipe ("CPU Overhead of te.Linear FP8 Layers": history 16,
algorithm "max").
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import exact


def _bf16(a32: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------- amax ----

@pytest.mark.parametrize("src", ["bf16", "fp32"])
def test_amax_brute_force(src):
    rng = np.random.default_rng(3)
    x32 = (rng.standard_normal((37, 53)) * 5).astype(np.float32)
    x32[5, 7] = -91.25
    x = _bf16(x32) if src == "bf16" else x32
    vals = oracle.bf16_bits_to_f32(x) if src == "bf16" else x32
    _, _, amax, _ = oracle.cast_transpose_amax(x, 1.0, oracle.E4M3)
    assert amax == np.max(np.abs(vals))
    # Accumulates with an incoming amax, and never decreases it.
    _, _, amax2, _ = oracle.cast_transpose_amax(x, 1.0, oracle.E4M3, amax_in=1000.0)
    assert amax2 == 1000.0
    _, _, amax3, _ = oracle.cast_transpose_amax(x, 1.0, oracle.E4M3, amax_in=0.5)
    assert amax3 == amax


def test_amax_is_of_the_unscaled_source():
    x = np.array([[3.0, -7.5, 0.25]], dtype=np.float32)
    _, _, amax, sinv = oracle.cast_transpose_amax(x, 1024.0, oracle.E4M3)
    assert amax == 7.5
    assert sinv == np.float32(1.0 / 1024.0)


def test_amax_special_values():
    def amax_of(vals):
        return oracle.cast_transpose_amax(np.array([vals], dtype=np.float32), 1.0, oracle.E5M2)[2]
    assert amax_of([-0.0, 0.0]) == 0.0
    assert amax_of([1e-45, -2e-45]) == np.float32(2e-45)          # fp32 subnormals kept
    assert np.isinf(amax_of([1.0, -np.inf, 3.0]))
    assert np.isnan(amax_of([1.0, np.inf, np.nan, 3.0]))
    assert np.isnan(amax_of([np.nan, -np.inf]))


def test_transpose_is_numpy_transpose():
    rng = np.random.default_rng(4)
    x = _bf16(rng.standard_normal((48, 80)).astype(np.float32))
    q, qt, _, _ = oracle.cast_transpose_amax(x, 3.0, oracle.E5M2)
    np.testing.assert_array_equal(qt, np.transpose(q))
    q2, qt2, _, _ = oracle.cast_transpose_amax(x, 3.0, oracle.E5M2, want_q=False)
    assert q2 is None
    np.testing.assert_array_equal(qt2, qt)


def test_scaled_cast_matches_exact_rounding():
    """v = fp32(x)*scale is one fp32 multiply: compare with exact rational math."""
    rng = np.random.default_rng(5)
    x = _bf16(rng.standard_normal((16, 16)).astype(np.float32))
    scale = np.float32(447.0 / 3.1)
    q, _, _, _ = oracle.cast_transpose_amax(x, float(scale), oracle.E4M3)
    t = oracle.decode_table(oracle.E4M3)
    code = {t[c]: c for c in range(128) if np.isfinite(t[c])}
    for xi, qi in zip(oracle.bf16_bits_to_f32(x).reshape(-1), q.reshape(-1)):
        v = exact.to_f32(exact.f32_fraction(xi) * exact.f32_fraction(scale))
        a = abs(Fraction(float(v)))
        want = 0x7E if a >= 448 else code[float(exact.round_binary(a, 4, -6))]
        assert qi == (want | (0x80 if v < 0 or (v == 0 and np.signbit(v)) else 0))


# --------------------------------------------------------- scale update ----

def _state(T, H=16):
    return (np.zeros((T, H), np.float32), np.zeros(T, np.float32), np.ones(T, np.float32),
            np.ones(T, np.float32))


def test_scale_closed_forms():
    amaxes = [1.0, 448.0, 2.0 ** -3, 2.0 ** 5, 57344.0, 1.0, 2.0 ** -10]
    fmts = [0, 0, 0, 0, 1, 1, 1]
    T = len(amaxes)
    hist, cur, scale, sinv = _state(T)
    cur[:] = amaxes
    fmt = np.array(fmts, np.uint8)
    oracle.scale_update(hist, cur, scale, sinv, fmt)
    want = [448.0, 1.0, 448.0 * 8, 448.0 / 32, 1.0, 57344.0, 57344.0 * 1024]
    assert list(scale) == want
    # amax = 2^k (E4M3) gives 1.75 * 2^(8-k) exactly.
    assert scale[3] == 1.75 * 2.0 ** (8 - 5)
    assert list(sinv) == [np.float32(1) / np.float32(s) for s in want]
    assert list(cur) == [0.0] * T
    assert list(hist[:, 0]) == amaxes and not hist[:, 1:].any()


def test_scale_margin():
    hist, cur, scale, sinv = _state(2)
    cur[:] = [1.0, 1.0]
    oracle.scale_update(hist, cur, scale, sinv, np.zeros(2, np.uint8), margin=1)
    assert list(scale) == [224.0, 224.0]
    hist, cur, scale, sinv = _state(1)
    cur[:] = [1.0]
    oracle.scale_update(hist, cur, scale, sinv, np.zeros(1, np.uint8), margin=-2)
    assert scale[0] == 448.0 * 4


def test_scale_non_power_of_two_is_correctly_rounded():
    rng = np.random.default_rng(8)
    amax = (rng.uniform(0.01, 1000, 64)).astype(np.float32)
    fmt = rng.integers(0, 2, 64).astype(np.uint8)
    hist, cur, scale, sinv = _state(64)
    cur[:] = amax
    oracle.scale_update(hist, cur, scale, sinv, fmt)
    for a, f, s, si in zip(amax, fmt, scale, sinv):
        fmax = 448 if f == 0 else 57344
        want = exact.to_f32(Fraction(fmax) / exact.f32_fraction(a))
        assert s == want
        assert si == exact.to_f32(1 / exact.f32_fraction(want))


def test_history_window_is_16_and_max():
    """An amax leaves the window after exactly 16 further updates."""
    H = 16
    hist, cur, scale, sinv = _state(1, H)
    fmt = np.zeros(1, np.uint8)
    seq = [100.0] + [1.0] * 16 + [0.5]
    scales = []
    for a in seq:
        cur[0] = a
        oracle.scale_update(hist, cur, scale, sinv, fmt)
        scales.append(float(scale[0]))
    want_first = float(exact.to_f32(Fraction(448) / 100))
    assert scales[:16] == [want_first] * 16     # 100 still in the 16-deep window
    assert scales[16] == 448.0                  # the 17th update evicts it
    assert scales[17] == 448.0                  # max over window, not the newest (0.5)
    assert list(hist[0]) == [0.5] + [1.0] * 15


def test_zero_or_nonfinite_amax_keeps_scale():
    hist, cur, scale, sinv = _state(4)
    scale[:] = [3.0, 5.0, 7.0, 9.0]
    cur[:] = [0.0, np.inf, np.nan, 1e-44]   # last: quotient overflows fp32
    oracle.scale_update(hist, cur, scale, sinv, np.zeros(4, np.uint8))
    assert list(scale) == [3.0, 5.0, 7.0, 9.0]
    assert list(sinv) == [np.float32(1) / np.float32(v) for v in (3.0, 5.0, 7.0, 9.0)]
    assert not cur.any()


def test_scale_update_rejects_bad_args():
    hist, cur, scale, sinv = _state(1)
    with pytest.raises(ValueError):
        oracle.scale_update(hist, cur, scale, sinv, np.array([2], np.uint8))
    with pytest.raises(ValueError):
        oracle.scale_update(hist, cur, scale, sinv, np.zeros(1, np.uint8), algo=1)
