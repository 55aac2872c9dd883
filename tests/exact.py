"""Exact rational helpers for pinning the oracle (pure Python, tiny inputs).

These are written from IEEE-754 definitions with ``fractions.Fraction`` and
share nothing with the oracle's C code: a value is rounded to p significant
bits by scaling it to an integer significand and breaking ties to even.
"""
from fractions import Fraction
import struct


def f32_bits_to_fraction(u: int) -> Fraction:
    f = struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]
    return Fraction(f)


def bf16_bits_to_fraction(h: int) -> Fraction:
    return f32_bits_to_fraction((h & 0xFFFF) << 16)


def _round_significand(v: Fraction, p: int, emin: int) -> Fraction:
    """Round v to p significant bits, nearest-even; quantum floored at 2^(emin-p+1)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e, emin) - (p - 1)              # quantum exponent
    scaled = a / (Fraction(2) ** q)
    fl = scaled.numerator // scaled.denominator
    rem = scaled - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * (Fraction(2) ** q)


def round_to_f32(v: Fraction) -> Fraction:
    """binary32: 24 significant bits, normals from 2^-126 (no overflow handling)."""
    return _round_significand(v, 24, -126)


def round_to_bf16(v: Fraction) -> Fraction:
    """bf16: 8 significant bits, normals from 2^-126 (no overflow handling)."""
    return _round_significand(v, 8, -126)


def fraction_to_bf16_bits(v: Fraction) -> int:
    """Bits of a value that is exactly representable in bf16 (finite)."""
    f = float(v)
    u = struct.unpack("<I", struct.pack("<f", f))[0]
    assert (u & 0xFFFF) == 0, "value is not a bf16"
    assert Fraction(f) == v
    return u >> 16
