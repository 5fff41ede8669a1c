"""Exact rational models of IEEE rounding, used to pin the oracle.

Everything here works on ``fractions.Fraction`` values and integer arithmetic
only; it shares nothing with the oracle's numpy code paths.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction


def f32(x: float) -> float:
    """The float32 value nearest to the Python float x (via struct, RNE)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def floor_log2(a: Fraction) -> int:
    """floor(log2 a) for a > 0, exactly."""
    assert a > 0
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # now 2^(e-1) < a < 2^(e+1); fix up
    if a >= Fraction(2) ** (e + 1):
        e += 1
    while a < Fraction(2) ** e:
        e -= 1
    return e


def rne_int(q: Fraction) -> int:
    """Round a rational to the nearest integer, ties to even."""
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl + (fl & 1)


def round_binary(q: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Round a rational to the nearest binary floating-point number with
    ``mant_bits`` significand bits (incl. the implicit one) and minimum normal
    exponent ``emin`` (gradual underflow), ties to even.  No overflow model."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(floor_log2(a), emin)
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    k = rne_int(a / ulp)
    return sign * k * ulp


def rn_f32(q: Fraction) -> Fraction:
    return round_binary(q, 24, -126)


def rn_bf16(q: Fraction) -> Fraction:
    return round_binary(q, 8, -126)


def int4_group(values):
    """Exact replay of the INT4 group quantizer on a list of floats.
    Returns (scale Fraction, list of int codes)."""
    vals = [Fraction(v) for v in values]
    a = max(abs(v) for v in vals)
    s = rn_f32(a / 7)
    if s == 0:
        return s, [0] * len(vals)
    codes = [max(-8, min(7, rne_int(rn_f32(v / s)))) for v in vals]
    return s, codes


E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
        Fraction(3), Fraction(4), Fraction(6)]


def e2m1_index(y: Fraction) -> int:
    """Nearest E2M1 magnitude index to |y|, ties to the even index."""
    a = abs(y)
    best = None
    for i, g in enumerate(E2M1):
        d = abs(a - g)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def fp4_block(values):
    """Exact replay of the E2M1/E8M0 block quantizer on a list of floats.
    Returns (scale byte, list of 4-bit sign-magnitude codes)."""
    vals = [Fraction(v) for v in values]
    a = max(abs(v) for v in vals)
    e = -127 if a == 0 else max(-127, min(127, floor_log2(a) - 2))
    codes = []
    for v, raw in zip(vals, values):
        y = v * Fraction(2) ** (-e)
        sign = 1 if math.copysign(1.0, raw) < 0 else 0
        codes.append((sign << 3) | e2m1_index(y))
    return e + 127, codes
