"""The GPTQ in-block kernel rounds x / s through y = RN(1/s): q0 = RN(x y),
r = x - s q0 (exact in one fused multiply-add), q = RN(q0 + r y).  By Markstein's theorem
on division by a correctly rounded reciprocal, q is the correctly rounded quotient, so
the codes equal those of the IEEE division.  This checks the identity in binary32 on the
values the kernel meets (weights near code boundaries, grid scales), emulating each
rounding exactly (host arithmetic only; no GPU)."""
from fractions import Fraction

import numpy as np


def _rn32(x: Fraction) -> np.float32:
    """Round an exact rational to the nearest binary32, ties to even."""
    f = np.float32(float(x))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - x),
                                     int(np.array(c, np.float32).view(np.int32)) & 1))


def _corrected_quotient(x: np.float32, s: np.float32) -> np.float32:
    y = np.float32(np.float32(1.0) / s)               # IEEE division: RN(1/s)
    q0 = np.float32(x * y)                            # RN(x y)
    r = _rn32(Fraction(float(x)) - Fraction(float(s)) * Fraction(float(q0)))
    return _rn32(Fraction(float(q0)) + Fraction(float(r)) * Fraction(float(y)))


def test_corrected_reciprocal_quotient_is_the_ieee_quotient():
    rng = np.random.default_rng(0)
    n = 6000
    s = rng.uniform(1e-3, 0.2, n).astype(np.float32)
    k = rng.integers(-8, 9, n).astype(np.float32)
    frac = rng.choice(np.array([0.5, 0.4999999, 0.5000001, 0.25, 0.0], np.float32), n)
    near = ((k + frac) * s).astype(np.float32)        # near rounding boundaries of x / s
    plain = (rng.standard_normal(n) * 0.05).astype(np.float32)
    for xs in (near, plain):
        for x, sv in zip(xs, s):
            assert _corrected_quotient(x, sv) == np.float32(x / sv), (x, sv)


def test_corrected_reciprocal_quotient_exact_cases():
    # exact quotients, powers of two and a zero numerator come out unchanged
    for x, s in ((0.75, 0.25), (-1.5, 0.5), (0.0, 0.1), (3.0, 0.375), (1e-3, 2.0 ** -7)):
        x32, s32 = np.float32(x), np.float32(s)
        assert _corrected_quotient(x32, s32) == np.float32(x32 / s32)
