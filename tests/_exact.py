"""Exact rational helpers for the oracle pins (independent of the oracle's C code).

Rounding here is done on Python Fractions, so it has no binary64 step at all;
the oracle rounds a binary64 value with frexp/nearbyint. Agreement between the
two pins the oracle's conversions.
"""
from fractions import Fraction

import mpmath
import numpy as np

# (significant bits, minimum normal exponent, largest finite value)
FORMATS = {
    "f16": (11, -14, Fraction(65504)),
    "bf16": (8, -126, Fraction(255) * Fraction(2) ** 120),
    "f32": (24, -126, Fraction(2 ** 24 - 1) * Fraction(2) ** 104),
}


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_ne(y: Fraction, fmt: str):
    """Nearest value of format `fmt` to the exact rational y, ties to even.

    Returns a float (possibly +-inf) that is exactly representable in `fmt`;
    a zero result carries the sign of y.
    """
    prec, emin, maxfin = FORMATS[fmt]
    if y == 0:
        return 0.0
    neg = y < 0
    a = -y if neg else y
    e = max(_floor_log2(a), emin)
    q = Fraction(2) ** (e - prec + 1)
    r = round(a / q) * q  # Fraction rounding is ties-to-even
    if r > maxfin:
        v = float("inf")
    else:
        v = float(r)  # exact: r has <= prec bits
    return -v if neg else v


def bits_of(v: float, fmt: str) -> int:
    """Storage bits of a value already exactly representable in fmt."""
    if fmt == "f16":
        return int(np.array(v, np.float16).view(np.uint16))
    if fmt == "bf16":
        return int(np.array(v, np.float32).view(np.uint32)) >> 16
    return int(np.array(v, np.float32).view(np.uint32))


def value_of(bits: int, fmt: str) -> Fraction:
    if fmt == "f16":
        return Fraction(float(np.array(bits, np.uint16).view(np.float16)))
    if fmt == "bf16":
        return Fraction(float(np.array(bits << 16, np.uint32).view(np.float32)))
    return Fraction(float(np.array(bits, np.uint32).view(np.float32)))


def rn24_mp(x) -> float:
    """mpmath value rounded once to float32 (nearest-even), as a Python float."""
    with mpmath.workprec(24):
        r = +x
    return float(r)


def near_f32_midpoint(x, slack_ulps53: int = 4) -> bool:
    """True if mpmath value x lies within a few binary64 ulps of a float32 midpoint
    (where rounding via binary64 may legitimately differ from direct rounding)."""
    with mpmath.workprec(200):
        lo = rn24_mp(x)
        # float32 spacing around lo
        e = _floor_log2(abs(Fraction(lo))) if lo != 0 else -126
        ulp = mpmath.mpf(2) ** (max(e, -126) - 23)
        mids = [mpmath.mpf(lo) + ulp / 2, mpmath.mpf(lo) - ulp / 2]
        tol = abs(x) * mpmath.mpf(2) ** (-53) * slack_ulps53
        return any(abs(x - m) <= tol for m in mids)
