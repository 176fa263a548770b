"""Exact rational rounding helpers used by the oracle pins.

IEEE binary32 / binary16 round-to-nearest-even of an exact rational, written
from the format definitions (precision p, minimum normal exponent emin,
subnormals below it). No numpy: these are an independent route to the values
the oracle must produce.
"""
from fractions import Fraction
import math
import struct

F32 = (24, -126, 127)    # precision, emin, emax
F16 = (11, -14, 15)


def rn(x, fmt=F32):
    """Round an exact rational to the nearest value of the format, ties to even.
    Returns a Fraction, or +-inf (float) on overflow."""
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    p, emin, emax = fmt
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix floating log2 errors
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (p - 1))
    q = a / ulp
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * ulp
    maxv = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if v > maxv:
        return sign * math.inf
    return sign * v


def f32_bits(v):
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def f16_bits(v):
    return struct.unpack("<H", struct.pack("<e", float(v)))[0]


def rint_even(x):
    """Round a rational to the nearest integer, ties to even."""
    x = Fraction(x)
    n = math.floor(x)
    r = x - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n
