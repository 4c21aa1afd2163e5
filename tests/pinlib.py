"""Exact-arithmetic helpers used to pin the oracle (test code only).

Nothing here is shared with the oracle or the HIP library: it models IEEE
binary32 rounding with Python ``fractions`` so that the oracle's float32
quantizer can be checked against arithmetic with no rounding of its own.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np

_TWO = Fraction(2)


def f32_round(x: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 value, ties to even.

    Handles normal and subnormal results (no overflow handling: callers stay
    far below 2^128).
    """
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if _TWO ** e > a:
        e -= 1
    while _TWO ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                   # below 2^-126 the spacing stays 2^-149
    quantum = _TWO ** (e - 23)
    m = a / quantum
    n = math.floor(m)
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * quantum


def f32_bits(x: Fraction) -> int:
    """IEEE binary32 bit pattern of an exactly representable value."""
    f = float(x)                       # exact: x is a binary32 value
    return struct.unpack("<I", struct.pack("<f", f))[0]


def frac_of_f32(v) -> Fraction:
    return Fraction(float(np.float32(v)))


def round_half_even(x: Fraction) -> int:
    n = math.floor(x)
    rem = x - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def exact_group_quantize(group_vals, bits: int):
    """Quantize one group with exact rationals and explicit binary32 rounding.

    Returns (scale as Fraction, list of signed codes q).
    """
    vals = [frac_of_f32(v) for v in group_vals]
    nh = (1 << (bits - 1)) - 1
    a = max(abs(v) for v in vals)                           # exact
    c101 = f32_round(Fraction(101, 100))                    # binary32 nearest 1.01
    a1 = f32_round(a * c101)
    step = f32_round(2 * a1 / ((1 << bits) - 1))
    if step == 0:
        return step, [0] * len(vals)
    qs = []
    for v in vals:
        r = f32_round(v / step)
        q = max(-nh, min(nh, round_half_even(r)))
        qs.append(q)
    return step, qs


def nearest_level(v: Fraction, step: Fraction, nh: int):
    """Brute force: the code in [-nh, nh] whose level q*step is nearest to v
    (ties to the even code), plus the distance from v/step to the nearest tie."""
    best = None
    for q in range(-nh, nh + 1):
        d = abs(v - q * step)
        key = (d, q % 2)
        if best is None or key < best[0]:
            best = (key, q)
    ratio = v / step
    tie_dist = abs(ratio - (math.floor(ratio) + Fraction(1, 2)))
    return best[1], tie_dist
