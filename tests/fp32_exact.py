"""Exact-rational binary32 arithmetic for pinning the oracle (test helper).

A third implementation, independent of both the C oracle and the GPU path:
values are Python ``Fraction``s and every result is rounded once, to the
nearest binary32 with ties to even, with gradual underflow (subnormals) and
overflow to infinity, as IEEE 754 defines for binary32 with
round-to-nearest-even. Python 3.10 has no ``math.fma``, and emulating a fused
multiply-add through double would round twice, hence the exact route.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

_EMIN = -126          # smallest normal exponent
_P = 24               # precision in bits (with the hidden bit)
_EMAX = 127


def _round_half_even(q: Fraction) -> int:
    """Nearest integer to a non-negative rational, ties to even."""
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def _floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # 2^e is within a factor of 2 of a; adjust once either way
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_f32(q: Fraction, zero_sign: int = 1) -> np.float32:
    """Round an exact rational to binary32 (RNE). ``zero_sign`` gives the sign
    of an exact zero (+1 or -1)."""
    if q == 0:
        return np.float32(0.0) if zero_sign > 0 else np.float32(-0.0)
    sign = -1 if q < 0 else 1
    a = -q if q < 0 else q
    e = max(_floor_log2(a), _EMIN)          # subnormals share the minimum exponent
    m = _round_half_even(a * Fraction(2) ** (_P - 1 - e))
    if m == 2 ** _P:                         # rounding carried into the next binade
        m //= 2
        e += 1
    if e > _EMAX:
        return np.float32(sign * np.inf)
    # m < 2**24 and 2**(e-23) is within double range: the product is exact
    return np.float32(sign * float(m) * 2.0 ** (e - (_P - 1)))


def fma_f32(a, b, c) -> np.float32:
    """Correctly rounded binary32 fused multiply-add a*b + c of finite inputs."""
    a, b, c = (np.float32(v) for v in (a, b, c))
    exact = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))
    if exact == 0:
        # IEEE: an exact zero sum of opposite-signed terms is +0 under RNE; the
        # sum of two zeros of the same sign keeps that sign.
        prod_neg = (np.signbit(a) != np.signbit(b))
        both_neg = prod_neg and bool(np.signbit(c)) and float(c) == 0.0 \
            and (float(a) == 0.0 or float(b) == 0.0)
        return round_f32(exact, -1 if both_neg else 1)
    return round_f32(exact)


def bits(x) -> int:
    return int(np.array(x, dtype=np.float32).view(np.uint32))
