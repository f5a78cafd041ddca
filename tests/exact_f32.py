"""Exact-rational binary32 arithmetic for the oracle's pins.

Nothing here calls the oracle or the HIP library. Rounding is done from the
exact rational value (fractions.Fraction) to binary32 with round-to-nearest,
ties-to-even, gradual underflow and overflow to infinity (IEEE 754-2008,
4.3.1 and 7.4), so a fused multiply-add computed here is correct by
construction rather than by trusting a library's fmaf.
"""
import math
from fractions import Fraction

import numpy as np

_MANT = 23          # stored mantissa bits of binary32
_EMIN = -126        # smallest normal exponent
_EMAX_PLUS1 = 128   # 2^128 is the overflow threshold after rounding


def f32_of_fraction(q):
    """Round the exact rational q to the nearest binary32 (ties to even)."""
    if q == 0:
        return np.float32(0.0)
    neg = q < 0
    a = -q if neg else q
    num, den = a.numerator, a.denominator
    e = num.bit_length() - den.bit_length()          # floor(log2 a) or one more
    if e >= 0:
        if num < (den << e):
            e -= 1
    elif (num << -e) < den:
        e -= 1
    qexp = max(e, _EMIN) - _MANT                       # exponent of one ulp
    if qexp >= 0:
        sn, sd = num, den << qexp
    else:
        sn, sd = num << -qexp, den
    m, rem = divmod(sn, sd)
    if 2 * rem > sd or (2 * rem == sd and (m & 1)):
        m += 1
    if m and qexp + m.bit_length() - 1 >= _EMAX_PLUS1:
        v = math.inf
    else:
        v = math.ldexp(m, qexp)
    return np.float32(-v if neg else v)


def frac(v):
    """Exact rational value of a finite float32 / float."""
    return Fraction(float(v))


def fma(a, b, c):
    """fmaf(a, b, c) for finite binary32 a, b, c, rounded once."""
    return f32_of_fraction(frac(a) * frac(b) + frac(c))


def add(a, b):
    return f32_of_fraction(frac(a) + frac(b))


def mul(a, b):
    return f32_of_fraction(frac(a) * frac(b))


def div(a, b):
    return f32_of_fraction(frac(a) / frac(b))


def sqrt(a):
    """Correctly rounded binary32 square root of a finite a >= 0, by exact
    integer search: r is the binary32 nearest to sqrt(a)."""
    if a == 0:
        return np.float32(a)
    q = frac(a)
    r0 = np.float32(math.sqrt(float(a)))        # within an ulp; fixed exactly below
    lo = np.nextafter(r0, np.float32(0))
    hi = np.nextafter(r0, np.float32(np.inf))
    for cand in (lo, r0, hi):
        below = np.nextafter(cand, np.float32(0))
        above = np.nextafter(cand, np.float32(np.inf))
        mlo = (frac(below) + frac(cand)) / 2
        mhi = (frac(cand) + frac(above)) / 2
        if mlo * mlo <= q <= mhi * mhi:
            # a tie (q exactly a midpoint squared) cannot occur: a midpoint
            # has 25 significant bits, its square is not a binary32 value.
            return cand
    raise AssertionError("sqrt: no binary32 within the midpoints")
