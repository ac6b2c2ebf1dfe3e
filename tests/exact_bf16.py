"""Exact bf16 helpers for the oracle's pins, written independently of the oracle.

Rounding here is "nearest representable value, ties to the even bit pattern",
found by a binary search over bf16 bit patterns with exact rational values.
The oracle instead scales by a power of two and rounds to an integer; the two
methods share nothing.
"""
from fractions import Fraction

MAX_FINITE = 0x7F7F
POS_INF = 0x7F80


def value(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern."""
    bits = int(bits) & 0xFFFF
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    assert e != 0xFF, "not finite"
    if e == 0:
        mag = Fraction(m, 1) * Fraction(1, 2 ** 133)
    else:
        mag = Fraction(128 + m) * (Fraction(2) ** (e - 127 - 7))
    return sign * mag


def rne_bits(x: Fraction) -> int:
    """bf16 bit pattern nearest to the rational x, ties to the even pattern."""
    x = Fraction(x)
    neg = x < 0
    a = -x if neg else x
    sign = 0x8000 if neg else 0
    # beyond the midpoint between the largest finite value and 2^128: infinity
    if a >= (value(MAX_FINITE) + Fraction(2) ** 128) / 2:
        return sign | POS_INF
    lo, hi = 0, MAX_FINITE          # largest pattern p with value(p) <= a
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if value(mid) <= a:
            lo = mid
        else:
            hi = mid - 1
    p = lo
    if p == MAX_FINITE or value(p) == a:
        return sign | p
    q = p + 1
    dp, dq = a - value(p), value(q) - a
    if dp < dq:
        return sign | p
    if dq < dp:
        return sign | q
    return sign | (p if p % 2 == 0 else q)


def bits_to_float(bits: int) -> float:
    return float(value(bits))
