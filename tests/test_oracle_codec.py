"""Pins for the oracle's FP8 codec (CPU only).

Each test fixes the oracle to something outside itself: the finfo table and
the worked cast table printed in "Accelerating PyTorch Training Workloads with
FP8 -- Part 2" (tests/golden/), brute force over all 256 codes, exact rational
rounding (tests/exact.py), and torch's own CPU float8 conversion as an
independent library.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import exact

GOLD = os.path.join(os.path.dirname(__file__), "golden")
FMTS = {"float8_e4m3fn": oracle.E4M3, "float8_e5m2": oracle.E5M2}
TORCH_DT = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _finite_sorted_codes(fmt):
    """Non-negative finite codes in increasing order of value."""
    t = oracle.decode_table(fmt)
    codes = [c for c in range(0, 128) if np.isfinite(t[c])]
    assert all(t[a] < t[b] for a, b in zip(codes, codes[1:])), "codes must be monotone"
    return codes, t


# ---------------------------------------------------------------- finfo ----

@pytest.mark.parametrize("name", ["float8_e4m3fn", "float8_e5m2"])
def test_finfo_table(name):
    row = _load("fp8_finfo.json")["rows"][name]
    fmt = FMTS[name]
    t = oracle.decode_table(fmt)
    fin = t[np.isfinite(t)]
    assert fin.max() == row["max"]
    assert fin.min() == row["min"]
    normals = [t[c] for c in range(128) if np.isfinite(t[c]) and (c >> (3 if fmt == 0 else 2)) & 0x1F]
    smallest_normal = min(v for v in normals if v > 0)
    assert smallest_normal == pytest.approx(row["smallest_normal"], rel=1e-5)
    one = list(t).index(1.0)
    assert t[one + 1] - 1.0 == row["eps"]
    assert oracle.fp8_max(fmt) == row["max"]


def test_finfo_pins_ocp_not_fnuz():
    # An FNUZ E4M3 (bias 8) would give max 240; an FNUZ E5M2 smallest normal 2^-15.
    assert np.nanmax(oracle.decode_table(oracle.E4M3)) == 448.0
    t5 = oracle.decode_table(oracle.E5M2)
    assert t5[0x04] == 2.0 ** -14
    assert np.isinf(t5[0x7C]) and np.isinf(t5[0xFC]) and t5[0xFC] < 0
    assert np.isnan(t5[0x7D]) and np.isnan(t5[0x7F])
    t4 = oracle.decode_table(oracle.E4M3)
    assert np.isnan(t4[0x7F]) and np.isnan(t4[0xFF])
    assert int(np.isnan(t4).sum()) == 2 and int(np.isnan(t5).sum()) == 6
    assert t4[0x80] == 0.0 and math.copysign(1, t4[0x80]) < 0


def test_bf16_finfo_row_pins_bf16_rounding():
    row = _load("fp8_finfo.json")["rows"]["bfloat16"]
    # Largest finite bf16 and machine epsilon.
    assert float(oracle.bf16_bits_to_f32(0x7F7F)) == pytest.approx(row["max"], rel=1e-5)
    one = oracle.f64_to_bf16_bits(1.0)
    assert float(oracle.bf16_bits_to_f32(one + 1)) - 1.0 == row["eps"]
    # 1 + eps/2 is a tie between 1 and 1+eps: even significand (1.0) wins.
    assert oracle.f64_to_bf16_bits(1.0 + row["eps"] / 2) == one
    assert oracle.f64_to_bf16_bits(1.0 + row["eps"] * 0.75) == one + 1
    assert float(oracle.bf16_bits_to_f32(0x0080)) == pytest.approx(row["smallest_normal"], rel=1e-5)


# --------------------------------------------------------- worked casts ----

def test_worked_cast_table_fp32_source():
    g = _load("worked_casts.json")
    x = np.array(g["float32"], dtype=np.float32)
    for name, fmt in FMTS.items():
        q = oracle.fp8_encode(x, fmt)
        assert list(oracle.fp8_decode(q, fmt)) == g[name], name


def test_worked_cast_table_bf16_row():
    g = _load("worked_casts.json")
    b = oracle.f64_to_bf16_bits(np.array(g["float32"], dtype=np.float32).astype(np.float64))
    got = oracle.bf16_bits_to_f32(b)
    np.testing.assert_allclose(got, g["bfloat16"], rtol=0, atol=5e-8)


def test_bf16_source_of_worked_value_is_a_tie():
    # -0.78251332044 rounds to bf16 -0.78125 = -(0.75 + 0.875)/2: an exact E4M3
    # tie between -0.75 (mantissa 100, even) and -0.8125 (101): RNE picks -0.75.
    b = oracle.f64_to_bf16_bits(np.float64(np.float32(-0.78251332044)))
    assert float(oracle.bf16_bits_to_f32(b)) == -0.78125
    q, _, _, _ = oracle.cast_transpose_amax(np.array([[b]], dtype=np.uint16), 1.0, oracle.E4M3)
    assert oracle.fp8_decode(q, oracle.E4M3)[0, 0] == -0.75


# ------------------------------------------------------- brute force 256 ----

@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_all_codes_round_trip(fmt):
    t = oracle.decode_table(fmt)
    n_finite = 0
    for c in range(256):
        v = t[c]
        if np.isnan(v):
            continue
        if np.isinf(v):
            # Saturating encoder: +-inf maps to +-max, never to the inf code.
            assert oracle.fp8_encode(np.float32(v), fmt) == (c & 0x80) | (0x7E if fmt == 0 else 0x7B)
            continue
        n_finite += 1
        assert oracle.fp8_encode(np.float32(v), fmt) == c, hex(c)
    assert n_finite == (254 if fmt == oracle.E4M3 else 248)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_midpoints_ties_to_even_and_neighbours(fmt):
    codes, t = _finite_sorted_codes(fmt)
    for lo, hi in zip(codes, codes[1:]):
        a, b = t[lo], t[hi]
        mid = np.float32((a + b) / 2)
        assert float(mid) == (a + b) / 2, "FP8 midpoints are exact in fp32"
        even = lo if lo % 2 == 0 else hi
        for sgn in (1, -1):
            sbit = 0 if sgn > 0 else 0x80
            assert oracle.fp8_encode(np.float32(sgn * mid), fmt) == sbit | even
            up = np.nextafter(mid, np.float32(np.inf), dtype=np.float32)
            dn = np.nextafter(mid, np.float32(0), dtype=np.float32)
            assert oracle.fp8_encode(np.float32(sgn * up), fmt) == sbit | hi
            assert oracle.fp8_encode(np.float32(sgn * dn), fmt) == sbit | lo


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_saturation_nan_and_zero(fmt):
    mx = oracle.fp8_max(fmt)
    maxcode = 0x7E if fmt == oracle.E4M3 else 0x7B
    for v in (mx, mx * 1.03, mx * 1.0625, mx * 1.5, 3.0e38, np.inf):
        assert oracle.fp8_encode(np.float32(v), fmt) == maxcode
        assert oracle.fp8_encode(np.float32(-v), fmt) == 0x80 | maxcode
    assert oracle.fp8_encode(np.float32(np.nan), fmt) == 0x7F
    assert oracle.fp8_encode(-np.float32(np.nan), fmt) == 0xFF
    assert oracle.fp8_encode(np.float32(0.0), fmt) == 0x00
    assert oracle.fp8_encode(np.float32(-0.0), fmt) == 0x80
    tiny = oracle.decode_table(fmt)[1]            # smallest subnormal
    assert oracle.fp8_encode(np.float32(tiny / 2), fmt) == 0x00       # tie -> even (0)
    assert oracle.fp8_encode(np.nextafter(np.float32(tiny / 2), np.float32(1)), fmt) == 0x01
    assert oracle.fp8_encode(np.float32(-1e-30), fmt) == 0x80
    assert oracle.fp8_encode(np.float32(1e-45), fmt) == 0x00          # fp32 subnormal


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_encode_against_exact_rational_rounding(fmt):
    """Random fp32 magnitudes across the whole FP8 range, rounded exactly."""
    p, emin = (4, -6) if fmt == oracle.E4M3 else (3, -14)
    t = oracle.decode_table(fmt)
    value_to_code = {t[c]: c for c in range(128) if np.isfinite(t[c])}
    rng = np.random.default_rng(11)
    e = rng.uniform(-20, 17 if fmt == oracle.E5M2 else 9.5, size=3000)
    v = (2.0 ** e * rng.choice([-1, 1], size=e.size)).astype(np.float32)
    mx = oracle.fp8_max(fmt)
    q = oracle.fp8_encode(v, fmt)
    for x, c in zip(v, q):
        a = abs(exact.f32_fraction(x))
        if a >= Fraction(mx):
            want = 0x7E if fmt == oracle.E4M3 else 0x7B
        else:
            r = exact.round_binary(a, p, emin)
            want = value_to_code[float(r)]
        want |= 0x80 if x < 0 else 0
        assert c == want, (float(x), hex(c), hex(want))


def _torch_ref(v32: np.ndarray, fmt: int) -> np.ndarray:
    """torch's CPU float8 conversion (an independent library encoder), with
    the input clamped to +-max first because torch's cast does not saturate."""
    mx = np.float32(oracle.fp8_max(fmt))
    c = np.clip(v32, -mx, mx)
    return torch.from_numpy(c).to(TORCH_DT[fmt]).view(torch.uint8).numpy()


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("scale", [1.0, 448.0, 0.0009765625, 3.3333333, 57344.0, 1.7e-3])
def test_all_bf16_patterns_against_torch(fmt, scale):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.reshape(256, 256)
    q, qt, amax, sinv = oracle.cast_transpose_amax(x, scale, fmt)
    with np.errstate(invalid="ignore", over="ignore"):
        v = (oracle.bf16_bits_to_f32(bits) * np.float32(scale)).astype(np.float32)
    ok = ~np.isnan(v)
    ref = _torch_ref(v[ok], fmt)
    np.testing.assert_array_equal(q.reshape(-1)[ok], ref)
    nanq = q.reshape(-1)[~ok]
    assert set(np.unique(nanq & 0x7F)) == {0x7F}
    np.testing.assert_array_equal(qt, q.T)
    assert np.isnan(amax)                 # bf16 NaN patterns are in the sweep
    assert sinv == np.float32(1.0) / np.float32(scale)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_random_fp32_patterns_against_torch(fmt):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=1 << 18, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    # Also concentrate samples where the FP8 grid lives.
    e = rng.uniform(-24, 20, size=1 << 17)
    v2 = (2.0 ** e * rng.standard_normal(e.size)).astype(np.float32)
    v = np.concatenate([v, v2])
    q = oracle.fp8_encode(v, fmt)
    np.testing.assert_array_equal(q, _torch_ref(v, fmt))


def test_nan_product_sign_rule():
    """A NaN product takes sign(x) XOR sign(scale); inf * 0 is such a NaN."""
    def code(x, scale, fmt=oracle.E4M3):
        q, _, _, _ = oracle.cast_transpose_amax(np.array([[x]], dtype=np.float32), scale, fmt)
        return int(q[0, 0])
    nan = np.float32(np.nan)
    assert code(nan, 2.0) == 0x7F and code(-nan, 2.0) == 0xFF
    assert code(nan, -2.0) == 0xFF and code(-nan, -2.0) == 0x7F
    assert code(np.inf, 0.0) == 0x7F and code(-np.inf, 0.0) == 0xFF
    assert code(0.0, np.inf, oracle.E5M2) == 0x7F and code(-0.0, np.inf, oracle.E5M2) == 0xFF
    assert code(1.0, nan) == 0x7F
    assert code(-1.0, -np.inf) == 0x7E and code(1.0, -np.inf, oracle.E5M2) == 0xFB
