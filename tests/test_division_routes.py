"""The GPU kernels reach three IEEE float32 results by cheaper exact routes; this
checks those routes in exact rational arithmetic on the CPU (no GPU, no oracle):

  * amax / 7:  q0 = RN(a * r7), e = RN(a - 7 q0) (exact, one fma),
               RN(q0 + e * r7) with r7 = RN(1/7)          (Markstein's correction);
               the same with 127 for the INT8 control's scale
  * 1 / s for an fp16-valued s: r0 = any float32 within one ulp of 1/s (the
               hardware reciprocal), e = RN(1 - s r0) (exact), RN(r0 + r0 e)
  * y / s:     q0 = RN(y * r), e = RN(y - s q0) (exact), RN(q0 + e r), r = RN(1/s)

Each must equal the correctly rounded quotient. Exact arithmetic with fractions;
fma(a, b, c) is modelled as one rounding of the exact a*b + c.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

from tests.exact_fp import F16, rn

R7 = Fraction(0x124925 | 0x800000, 1 << 26)      # float32 0x3E124925
R127 = Fraction(0x010204 | 0x800000, 1 << 30)    # float32 0x3C010204


def fma(a, b, c):
    return rn(a * b + c)


def ulp32(x):
    x = abs(Fraction(x))
    e = math.floor(math.log2(x.numerator) - math.log2(x.denominator))
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    return Fraction(2) ** (max(e, -126) - 23)


def test_r7_is_rn_of_one_seventh():
    assert R7 == rn(Fraction(1, 7))
    assert R127 == rn(Fraction(1, 127))


def div7_route(a):
    q0 = rn(a * R7)
    e = fma(-q0, Fraction(7), a)
    assert e == a - 7 * q0            # the residual is exact
    return fma(e, R7, q0)


def test_div7_route_is_correctly_rounded():
    rng = np.random.default_rng(0)
    cases = [Fraction(0), Fraction(7), Fraction(1, 1 << 20)]
    # every float32 significand pattern near the top, bottom and middle of a binade,
    # over binades from fp16-subnormal magnitudes up to the largest amax reachable
    for e in range(-27, 21):
        for m in list(range(0, 64)) + list(range((1 << 23) - 64, 1 << 23)) + \
                [int(v) for v in rng.integers(0, 1 << 23, 64)]:
            cases.append(Fraction((1 << 23) | m) * Fraction(2) ** (e - 23))
    for a in cases:
        assert div7_route(a) == rn(a / 7), a


def div127_route(a):
    q0 = rn(a * R127)
    e = fma(-q0, Fraction(127), a)
    assert e == a - 127 * q0
    return fma(e, R127, q0)


def test_div127_route_is_correctly_rounded():
    """amax / 127 for the INT8 control's scale, same sweep as for / 7."""
    rng = np.random.default_rng(5)
    cases = [Fraction(0), Fraction(127), Fraction(1, 1 << 20)]
    for e in range(-27, 21):
        for m in list(range(0, 64)) + list(range((1 << 23) - 64, 1 << 23)) + \
                [int(v) for v in rng.integers(0, 1 << 23, 64)]:
            cases.append(Fraction((1 << 23) | m) * Fraction(2) ** (e - 23))
    for a in cases:
        assert div127_route(a) == rn(a / 127), a


def fp16_values():
    """Every positive finite fp16 value, as exact fractions."""
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    return [Fraction(float(v)) for v in bits.view(np.float16)]


def test_reciprocal_route_all_fp16_scales():
    for s in fp16_values():
        want = rn(1 / s)
        u = ulp32(want)
        for r0 in (want - u, want, want + u):        # any faithful hardware reciprocal
            e = fma(-s, r0, Fraction(1))
            assert e == 1 - s * r0                     # exact
            assert fma(r0, e, r0) == want, (s, r0)


def test_quotient_route_near_half_integers():
    """y / s for a spread of fp16 scales and float32 y within a few ulps of every
    half-integer k + 1/2, k in [-9, 8] (the only places where the rounding to an
    integer code can go wrong), plus exact ties."""
    rng = np.random.default_rng(1)
    scales = fp16_values()
    pick = [scales[i] for i in rng.choice(len(scales), 120, replace=False)]
    pick += [Fraction(1), Fraction(65504), Fraction(1, 1 << 24), Fraction(3, 1 << 12)]
    for s in pick:
        r = rn(1 / s)
        for k in range(-9, 9):
            target = rn((Fraction(2 * k + 1, 2)) * s)
            u = ulp32(target) if target != 0 else Fraction(1, 1 << 149)
            for d in range(-3, 4):
                y = target + d * u
                q0 = rn(y * r)
                e = fma(-q0, s, y)
                assert e == y - s * q0
                assert fma(e, r, q0) == rn(y / s), (s, y)


# Single-fma code route of the INT4 append (fast path): t = RN(u * RN(c r) + kT)
# with kT = 136.5 + 2^-16, so that t lies in [128, 256) on the 2^-16 grid; the
# code is floor(t - 128) - 8 (byte 2 of t's bits) unless the low 16 bits of t
# are 0 or 1, which sends the wave to the exact route above. u is the
# un-normalised transform value, y = RN(c u) the rotated value (c = 1 without
# rotation), r = RN(1/s).
KT = Fraction(273, 2) + Fraction(1, 1 << 16)
C_H = {1: Fraction(1), 16: Fraction(1, 4), 64: Fraction(1, 8),
       32: Fraction(0x3504F3 | 0x800000, 1 << 26),        # float32 0x3E3504F3
       128: Fraction(0x3504F3 | 0x800000, 1 << 27)}       # float32 0x3DB504F3


def rint_even(x):
    n = math.floor(x)
    r = x - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def code_route(u, cr):
    t = rn(u * cr + KT)
    assert 128 <= t < 256
    n = (t - 128) * (1 << 16)
    assert n.denominator == 1
    n = n.numerator
    return (n >> 16) - 8, (n & 0xFFFF) <= 1


def test_c_h_constants_are_rn_of_inverse_sqrt():
    for h in (32, 128):
        c = C_H[h]
        assert rn(c) == c
        lo, hi = c - ulp32(c) / 2, c + ulp32(c) / 2
        assert lo * lo * h < 1 < hi * hi * h


def test_single_fma_route_flags_every_misrounding():
    """For fp16 scales s and rotated values y within a few ulps of every
    half-integer multiple of s (and random ones), every code the fast route
    does not flag equals rint(RN(y / s)); near-ties are flagged, random values
    rarely are."""
    rng = np.random.default_rng(7)
    scales = fp16_values()
    normal = [s for s in scales if s >= Fraction(1, 1 << 14)]
    pick = [normal[i] for i in rng.choice(len(normal), 24, replace=False)]
    pick += [Fraction(1, 1 << 14), Fraction(65504), Fraction(1), Fraction(3, 1 << 12)]
    flagged_near = total_near = flagged_rand = total_rand = 0
    for s in pick:
        r = rn(1 / s)
        for h, c in C_H.items():
            cr = rn(c * r)
            cases = []
            for k in range(-8, 8):
                target = rn(Fraction(2 * k + 1, 2) * s)
                for d in (-2, -1, 0, 1, 2):
                    y = target + d * ulp32(target)
                    u0 = rn(y / c)
                    for du in (-1, 0, 1):
                        cases.append((u0 + du * ulp32(u0), True))
            for v in rng.uniform(-7.0, 7.0, 40):
                cases.append((rn(Fraction(float(v)) * s / c), False))
            for u, near in cases:
                y = rn(c * u)
                if abs(y / s) > Fraction(7004, 1000):
                    continue
                want = max(-8, min(7, rint_even(rn(y / s))))
                code, flag = code_route(u, cr)
                if not flag:
                    assert code == want, (s, h, u)
                if near:
                    total_near += 1
                    flagged_near += flag
                else:
                    total_rand += 1
                    flagged_rand += flag
    assert flagged_near > total_near // 4
    assert flagged_rand * 100 < total_rand
