"""Exact-arithmetic brute force used to pin the oracle (test helper).

Everything here is written independently of oracle.c: exact rationals
(``fractions.Fraction``), 80-digit decimals for square roots, and nearest-value
searches over explicit candidate lists instead of any rounding formula.
"""
from __future__ import annotations

import struct
from decimal import Decimal, getcontext
from fractions import Fraction

getcontext().prec = 80


def bf16_exact(bits: int) -> Fraction:
    """Exact value of a finite BF16 pattern (the top half of a binary32)."""
    f = struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]
    return Fraction(f)


def _bf16_mag_guess(m: float) -> int:
    if m > 3.3e38:
        m = 3.3e38
    return struct.unpack("<I", struct.pack("<f", m))[0] >> 16


def _dec(x) -> Decimal:
    if isinstance(x, Decimal):
        return x
    if isinstance(x, Fraction):
        return Decimal(x.numerator) / Decimal(x.denominator)
    return Decimal(x)


def bf16_nearest(v) -> int:
    """BF16 pattern nearest to v (Fraction or Decimal), ties to the even
    pattern, found by comparing distances to the neighbouring candidates."""
    neg = v < 0
    m = -v if neg else v
    c0 = _bf16_mag_guess(float(m))
    cands = [c for c in range(c0 - 3, c0 + 4) if 0 <= c <= 0x7F7F]
    md = _dec(m)
    best, bd = None, None
    for c in cands:
        d = abs(_dec(bf16_exact(c)) - md)
        if bd is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    return best | (0x8000 if neg else 0)


def dec_sqrt(x) -> Decimal:
    return _dec(x).sqrt()


def e4m3_bits_value(c: int) -> float:
    """E4M3FN code -> value by building the binary32 bit pattern (sign, biased
    exponent, mantissa moved into place); NaN for S.1111.111."""
    s, E, M = (c >> 7) & 1, (c >> 3) & 15, c & 7
    if E == 15 and M == 7:
        return float("nan")
    if E == 0:
        # subnormal: M/8 * 2^-6 = M * 2^-9; build it from the integer
        val = float(M) * (2.0 ** -9)
    else:
        bits = ((E - 7 + 127) << 23) | (M << 20)
        val = struct.unpack("<f", struct.pack("<I", bits))[0]
    return -val if s else val


def e4m3_brute(y: float) -> int:
    """Nearest finite E4M3FN code to y by search over all codes of y's sign,
    saturating, ties to the even code."""
    neg = (y < 0) or (y == 0 and str(y).startswith("-"))
    base = 0x80 if neg else 0x00
    a = Fraction(abs(y)) if abs(y) != float("inf") else Fraction(10 ** 6)
    best, bd = None, None
    for m in range(0x7F):  # 0x00..0x7E: the finite magnitudes
        d = abs(Fraction(e4m3_bits_value(m)) - a)
        if bd is None or d < bd or (d == bd and m % 2 == 0):
            best, bd = m, d
    return base | best


def e4m3_brute_vec(y):
    """Vectorised e4m3_brute for float32 arrays (finite inputs).

    Distances are taken in float64; they are exact wherever a tie can occur,
    since a float32 input and the two codes around it lie within a factor of two
    of each other (or one of them is zero)."""
    import numpy as np
    y = np.asarray(y, dtype=np.float32)
    mags = np.array([e4m3_bits_value(m) for m in range(0x7F)], dtype=np.float64)
    # beyond 448 the nearest finite code is 448 itself; clamping keeps the
    # float64 distances exact for huge inputs
    a = np.minimum(np.abs(y.astype(np.float64)), 1000.0)
    d = np.abs(a[:, None] - mags[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    # among equal distances prefer the even code, then the smaller one
    codes = np.arange(0x7F)
    score = np.where(cand, (codes % 2) * 1000 + codes, 10 ** 9)
    best = score.argmin(axis=1).astype(np.uint8)
    neg = np.signbit(y)
    return np.where(neg, best | 0x80, best).astype(np.uint8)
