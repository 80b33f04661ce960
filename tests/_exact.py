"""Exact rational arithmetic for pinning the oracle (tests only).

Written independently of ``oracle/oracle.c``: bit fields are decoded with
Python integers and ``fractions.Fraction``, sums are exact, and rounding to
FP16 / BF16 is done on exact rationals.  Every finite FP16 value is an integer
multiple of 2^-24 and every finite BF16 value an integer multiple of 2^-133,
so these sums carry no rounding at all.
"""
from __future__ import annotations

from fractions import Fraction

FORMATS = {
    # name: (fraction bits, exponent bits, bias)
    "f16": (10, 5, 15),
    "bf16": (7, 8, 127),
}


def value(fmt: str, bits: int) -> Fraction:
    fb, eb, bias = FORMATS[fmt]
    sign = -1 if (bits >> 15) & 1 else 1
    e = (bits >> fb) & ((1 << eb) - 1)
    f = bits & ((1 << fb) - 1)
    if e == (1 << eb) - 1:
        raise ValueError("not finite")
    if e == 0:
        return sign * Fraction(f) * Fraction(2) ** (1 - bias - fb)
    return sign * Fraction((1 << fb) | f) * Fraction(2) ** (e - bias - fb)


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_bits(fmt: str, x: Fraction, negative_zero: bool = False) -> int:
    """Round-half-even of an exact rational to ``fmt``; overflow to infinity."""
    fb, eb, bias = FORMATS[fmt]
    emin = 1 - bias
    emax = (1 << eb) - 2 - bias
    sign = 0x8000 if (x < 0 or (x == 0 and negative_zero)) else 0
    a = abs(x)
    if a == 0:
        return sign
    E = max(_floor_log2(a), emin)
    q = Fraction(2) ** (E - fb)
    t = a / q
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * q
    inf = ((1 << eb) - 1) << fb
    if r >= Fraction(2) ** (emax + 1):
        return sign | inf
    if r < Fraction(2) ** emin:
        return sign | int(r / Fraction(2) ** (emin - fb))
    Er = _floor_log2(r)
    frac = int(r / Fraction(2) ** (Er - fb)) - (1 << fb)
    return sign | ((Er + bias) << fb) | frac


def gemm(layout: str, fmt: str, A, B):
    """Exact d[i][j] and s[i][j] (lists of Fractions) for small operands.

    ``A`` is M x K; ``B`` is N x K ("nt") or K x N ("nn"); entries are bit
    patterns (ints).
    """
    M, K = len(A), len(A[0]) if len(A) else 0
    N = len(B) if layout == "nt" else (len(B[0]) if len(B) else 0)
    av = [[value(fmt, int(A[i][k])) for k in range(K)] for i in range(M)]
    if layout == "nt":
        bv = [[value(fmt, int(B[j][k])) for k in range(K)] for j in range(N)]
    else:
        bv = [[value(fmt, int(B[k][j])) for k in range(K)] for j in range(N)]
    d = [[sum((av[i][k] * bv[j][k] for k in range(K)), Fraction(0)) for j in range(N)]
         for i in range(M)]
    s = [[sum((abs(av[i][k] * bv[j][k]) for k in range(K)), Fraction(0)) for j in range(N)]
         for i in range(M)]
    return d, s
