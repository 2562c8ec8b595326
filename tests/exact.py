"""Exact-arithmetic helpers for the tests (Python Fractions), independent of the
oracle's C code and of the HIP library."""
from __future__ import annotations

import struct
from fractions import Fraction

BF16_MAX = Fraction(0xFF, 0x80) * Fraction(2) ** 127  # 1.1111111b * 2^127


def round_half_even(x: Fraction) -> int:
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def frac_to_bf16_bits(x: Fraction, negative_zero: bool = False) -> int:
    """Exact value -> BF16 bits, one round-to-nearest-even (8 significant bits)."""
    if x == 0:
        return 0x8000 if negative_zero else 0
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2^e <= a < 2^(e+1)
    qexp = max(e - 7, -133)
    n = round_half_even(a / Fraction(2) ** qexp)
    v = Fraction(n) * Fraction(2) ** qexp
    if v > BF16_MAX:
        return sign | 0x7F80
    f = struct.unpack("<I", struct.pack("<f", float(v)))[0]
    assert Fraction(struct.unpack("<f", struct.pack("<I", f))[0]) == v
    return sign | (f >> 16)


def bf16_bits_to_frac(b: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0])


def f32_to_frac(x) -> Fraction:
    return Fraction(float(struct.unpack("<f", struct.pack("<f", float(x)))[0]))


def near_bf16_boundary(x: Fraction, rel: float = 2.0 ** -40) -> bool:
    """True if x lies within `rel` (relative) of a BF16 rounding boundary (a midpoint)."""
    if x == 0:
        return False
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = Fraction(2) ** max(e - 7, -133)
    t = a / q
    frac = t - (t.numerator // t.denominator)
    return abs(frac - Fraction(1, 2)) * q <= a * Fraction(rel)
