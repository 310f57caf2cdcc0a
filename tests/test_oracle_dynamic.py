"""Pins of the oracle's dynamic-scaling cast (the comparator of delayed
scaling on "support delayed scaling of weight in float8 all-gather"):
closed-form scales for power-of-two amaxes, the largest element landing on
the largest code, the guard cases, and numpy's max for the amax."""
import numpy as np

import oracle

MAXCODE = {oracle.E4M3: 0x7E, oracle.E5M2: 0x7B}
FP8_MAX = {oracle.E4M3: 448.0, oracle.E5M2: 57344.0}


def _bits(a):
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return (b >> 16).astype(np.uint16)


def test_power_of_two_amax_gives_exact_scale():
    rng = np.random.default_rng(1)
    for fmt in (oracle.E4M3, oracle.E5M2):
        for k in (-6, 0, 3):
            for margin in (0, 2):
                x = np.clip(rng.standard_normal((64, 48)), -1, 1).astype(np.float32) * 2.0 ** k * 0.9
                x[5, 7] = -(2.0 ** k)                       # amax, exact power of two
                _, _, amax, scale, sinv = oracle.dynamic_cast(_bits(x), fmt, margin=margin)
                assert amax == 2.0 ** k
                assert scale == np.float32(FP8_MAX[fmt] * 2.0 ** (-k - margin))
                assert sinv == np.float32(1.0) / scale


def test_amax_element_maps_to_max_code():
    rng = np.random.default_rng(2)
    for fmt in (oracle.E4M3, oracle.E5M2):
        x = (rng.standard_normal((128, 96)) * 3.7).astype(np.float32)
        q, qt, amax, scale, _ = oracle.dynamic_cast(x, fmt)
        assert amax == np.float32(np.abs(x).max())
        r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        assert (q[r, c] & 0x7F) == MAXCODE[fmt]
        assert (q[r, c] >> 7) == (1 if x[r, c] < 0 else 0)
        np.testing.assert_array_equal(qt, q.T)


def test_cast_uses_the_derived_scale():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 64)) * 0.01).astype(np.float32)
    q, qt, amax, scale, sinv = oracle.dynamic_cast(_bits(x), oracle.E5M2)
    cq, cqt, _, csinv = oracle.cast_transpose_amax(_bits(x), float(scale), oracle.E5M2)
    np.testing.assert_array_equal(q, cq)
    assert sinv == csinv


def test_guards_keep_the_fallback_scale():
    z = np.zeros((32, 32), np.uint16)
    q, _, amax, scale, sinv = oracle.dynamic_cast(z, oracle.E4M3, fallback_scale=7.0)
    assert amax == 0.0 and scale == 7.0 and sinv == np.float32(1 / 7.0) and (q == 0).all()
    x = np.ones((32, 32), np.float32)
    x[1, 1] = np.nan
    _, _, amax, scale, _ = oracle.dynamic_cast(x, oracle.E4M3, fallback_scale=3.0)
    assert np.isnan(amax) and scale == 3.0
    tiny = np.full((16, 16), 1e-45, np.float32)              # fp8_max / tiny overflows
    _, _, amax, scale, _ = oracle.dynamic_cast(tiny, oracle.E5M2, fallback_scale=5.0)
    assert amax > 0 and scale == 5.0
