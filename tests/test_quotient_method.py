"""The element-quotient form the quantiser uses on its fast path, checked in exact arithmetic.

Per 16-element block the device computes y = RN(1 / b) once and, for each element a,
q0 = RN(a y), r0 = RN(a - q0 b), q1 = RN(q0 + r0 y), r1 = RN(a - q1 b), q' = RN(q1 + r1 y)
(every RN(x - y z) and RN(x + y z) one fma), with b = s g the block's decode scale.  q0 can
be slightly more than one ulp from a / b; the first correction makes q1 a faithful
quotient (within one ulp), so r1 is exact and, y being the correctly rounded reciprocal,
Markstein's theorem on division with a fused multiply-add (Muller et al., Handbook of
Floating-Point Arithmetic) gives q' = RN(a / b): the E2M1 codes equal those of a plain
division.  This test recomputes every step with exact rationals and one binary32
round-to-nearest-even per step, checks the intermediate claims (q1 faithful, r1 exact) and
the result, on dividends placed on and within a few ulps of the E2M1 rounding thresholds and
on random dividends, for divisors drawn as (E4M3 scale) x (binary32 global scale) across the
range the device uses the form for.  It exercises the method only: neither the oracle nor
the library is involved.
"""
from fractions import Fraction

import numpy as np


def rn32(x: Fraction) -> Fraction:
    """Round a positive rational to the nearest binary32 value, ties to even (normal range)."""
    assert x > 0
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    assert Fraction(2) ** e <= x < Fraction(2) ** (e + 1)
    assert -126 <= e <= 127
    ulp = Fraction(2) ** (e - 23)
    m = x / ulp                       # in [2^23, 2^24)
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n * ulp


def f32(v) -> Fraction:
    return Fraction(float(np.float32(v)))


def bits_plus(v: Fraction, k: int) -> Fraction:
    u = np.array([float(v)], np.float32).view(np.int32) + np.int32(k)
    return Fraction(float(u.view(np.float32)[0]))


def e4m3_values():
    vals = [Fraction(c, 512) for c in range(1, 8)]
    for c in range(8, 127):
        vals.append(Fraction(8 + (c & 7), 8) * Fraction(2) ** ((c >> 3) - 7))
    return vals


THRESHOLDS = [Fraction(x) for x in ("0.25", "0.75", "1.25", "1.75", "2.5", "3.5", "5")]


def rn32_signed(x: Fraction) -> Fraction:
    return x if x == 0 else (rn32(x) if x > 0 else -rn32(-x))


def ulp32(x: Fraction) -> Fraction:
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    return Fraction(2) ** (e - 23)


def block_quotient(a: Fraction, b: Fraction) -> Fraction:
    y = rn32(1 / b)
    q0 = rn32(a * y)
    r0 = rn32_signed(a - q0 * b)
    q1 = rn32(q0 + r0 * y)
    assert abs(q1 - a / b) < ulp32(a / b)          # faithful after one correction
    r1_exact = a - q1 * b
    r1 = rn32_signed(r1_exact)
    assert r1 == r1_exact                          # so the remainder is exact
    return rn32(q1 + r1 * y)


def test_rn32_matches_numpy_on_representable_and_midpoints():
    rng = np.random.default_rng(3)
    for v in rng.uniform(0.1, 100.0, 200).astype(np.float32):
        fv = Fraction(float(v))
        assert rn32(fv) == fv
        up = bits_plus(fv, 1)
        mid = (fv + up) / 2
        even = fv if (np.array([v], np.float32).view(np.int32)[0] % 2 == 0) else up
        assert rn32(mid) == even


def test_reciprocal_fma_quotient_is_correctly_rounded():
    rng = np.random.default_rng(20240611)
    svals = e4m3_values()
    n_checked = 0
    for _ in range(1500):
        s = svals[rng.integers(len(svals))]
        g = f32(np.float32(2.0) ** rng.uniform(-60, 60))
        b = rn32(s * g)
        if not (Fraction(2) ** -100 <= b <= Fraction(2) ** 100):
            continue
        for t in THRESHOLDS:
            base = rn32(t * b)
            for k in range(-3, 4):
                a = bits_plus(base, k)
                assert block_quotient(a, b) == rn32(a / b), (float(a), float(b))
                n_checked += 1
        for _ in range(4):
            a = f32(float(b) * rng.uniform(0.0, 6.5))
            if a > 0:
                assert block_quotient(a, b) == rn32(a / b), (float(a), float(b))
                n_checked += 1
    assert n_checked > 20000
