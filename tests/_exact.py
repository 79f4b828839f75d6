"""Exact rational emulation of IEEE binary32 / bf16 rounding (test helper).

Independent of the oracle: values become ``fractions.Fraction``, additions
and multiplications are exact, and each result is rounded to the nearest
representable value of a binary format with ``p`` significand bits (ties to
even, gradual underflow, overflow to infinity when the rounded magnitude
reaches 2**(emax+1)).  Used to pin the oracle's numpy float32 arithmetic.
"""

import math
import struct
from fractions import Fraction

import numpy as np


def round_binary(q, p, emin=-126, emax=127):
    """Nearest binary value with p significand bits to the rational q."""
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(Fraction(q))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - p + 1)
    m = a / quantum
    n = math.floor(m)
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * quantum
    if r >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * float(r)


def f32_add(a, b):
    """binary32 a + b, exactly rounded, for Python floats holding f32 values."""
    if math.isinf(a) or math.isinf(b):
        return a + b
    s = Fraction(a) + Fraction(b)
    if s == 0:
        both_neg_zero = (a == 0 and math.copysign(1, a) < 0 and b == 0 and math.copysign(1, b) < 0)
        return -0.0 if both_neg_zero else 0.0
    return round_binary(s, 24)


def f32_mul(a, b):
    if math.isinf(a) or math.isinf(b):
        return a * b
    s = Fraction(a) * Fraction(b)
    if s == 0:
        neg = (math.copysign(1, a) * math.copysign(1, b)) < 0
        return -0.0 if neg else 0.0
    return round_binary(s, 24)


def to_bf16_bits(v):
    """Round a float (holding an f32 value) to bf16 and return its bit pattern."""
    if math.isnan(v):
        return 0x7FC0
    if math.isinf(v):
        r = v
    elif v == 0:
        r = v
    else:
        r = round_binary(Fraction(v), 8)
    return struct.unpack("<I", struct.pack("<f", r))[0] >> 16


def bf16_value(bits):
    return float(np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0])


def fold_bf16_exact(columns):
    """columns: list over ranks of bf16 bit patterns for ONE element."""
    s = bf16_value(columns[0])
    for b in columns[1:]:
        s = f32_add(s, bf16_value(b))
    return to_bf16_bits(s)
