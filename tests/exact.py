"""Exact rational rounding, used to pin the oracle independently of its own code.

Nothing here is shared with the oracle or with the GPU library: it is a second,
deliberately different route (Python ``Fraction`` arithmetic) to the values the
oracle must produce.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_binary(fr: Fraction, p: int, emin: int) -> Fraction:
    """Nearest value with p significand bits (implicit bit included) and
    smallest normal exponent emin (gradual underflow below it); ties to the
    even significand.  No overflow handling: the caller checks the range."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = max(floor_log2(a), emin)
    q = Fraction(2) ** (e - (p - 1))
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * q


def to_f32(fr: Fraction) -> np.float32:
    """Correctly rounded fp32 of an exact rational (overflow -> inf)."""
    r = round_binary(fr, 24, -126)
    if abs(r) >= Fraction(2) ** 128:
        return np.float32(np.inf if r > 0 else -np.inf)
    return np.float32(float(r))  # representable, so the conversions are exact


def to_bf16_bits(fr: Fraction) -> int:
    """Correctly rounded bf16 bit pattern of an exact rational (overflow -> inf)."""
    r = round_binary(fr, 8, -126)
    if abs(r) >= Fraction(2) ** 128:
        return 0x7F80 if r > 0 else 0xFF80
    bits = int(np.array([float(r)], dtype=np.float32).view(np.uint32)[0]) >> 16
    if r == 0 and fr < 0:
        bits = 0x8000
    return bits


def f32_fraction(x) -> Fraction:
    return Fraction(float(np.float32(x)))
