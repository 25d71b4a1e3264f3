"""Exact rational arithmetic for pinning the oracle's fp32 steps.

Nothing here calls the oracle or the GPU library.  IEEE 754 binary32
round-to-nearest-even is written out from the format's definition on
``fractions.Fraction`` values, so a float result of the oracle can be checked
against the exact real-number result of the same operation.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

_EMIN = -126          # smallest normal exponent of binary32
_P = 24               # binary32 precision (bits, implicit one included)
_MAX = (2 - Fraction(1, 2 ** 23)) * Fraction(2) ** 127


def _round_half_even(v: Fraction) -> int:
    fl = math.floor(v)
    rem = v - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def round_f32(v: Fraction) -> np.float32:
    """The binary32 value nearest to the rational v (ties to even), with overflow to inf."""
    if v == 0:
        return np.float32(0.0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum_exp = max(e, _EMIN) - (_P - 1)
    quantum = Fraction(2) ** quantum_exp
    n = _round_half_even(a / quantum)
    r = n * quantum
    if r > _MAX:
        return np.float32(sign * np.inf)
    return np.float32(sign * float(r))


def frac(x) -> Fraction:
    """Exact rational value of a finite float32/float64."""
    return Fraction(float(x))


def rint_half_even(v: Fraction) -> int:
    return _round_half_even(v)


def bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
