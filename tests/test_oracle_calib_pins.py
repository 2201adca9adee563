"""Pins of the oracle's calibration variants s = (column max)^(q/4): q = 4 is
the column maximum itself, q = 0 all ones, q = 2 the square-root scale the
layer uses, and q = 1 two correctly rounded square roots in turn (checked
with exact rationals against the half-ulp brackets of each step)."""
from fractions import Fraction

import numpy as np


def _next(v, d):
    return float(np.nextafter(np.float32(v), np.float32(d)))


def _is_rounded_sqrt(v: float, m: Fraction) -> bool:
    lo = (Fraction(v) + Fraction(_next(v, -np.inf))) / 2
    hi = (Fraction(v) + Fraction(_next(v, np.inf))) / 2
    return lo * lo <= m <= hi * hi


def _x():
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((48, 80)) * 5).astype(np.float32)
    x[:, 3] = 0.0
    x[7, 11] = -300.0
    return x


def test_calibrate_pow_closed_forms(orc):
    x = _x()
    mx = np.max(np.abs(x), axis=0)
    s4 = orc.calibrate_pow(x, 4)
    assert np.array_equal(s4, np.where(mx == 0, 1.0, mx).astype(np.float32))
    assert np.all(orc.calibrate_pow(x, 0) == 1.0)
    assert np.array_equal(orc.calibrate_pow(x, 2), orc.calibrate(x))


def test_calibrate_pow_quarter_is_two_rounded_roots(orc):
    x = _x()
    s2 = orc.calibrate_pow(x, 2)
    s1 = orc.calibrate_pow(x, 1)
    mx = np.max(np.abs(x), axis=0)
    for k in range(x.shape[1]):
        if mx[k] == 0:
            assert s1[k] == 1.0
            continue
        assert _is_rounded_sqrt(float(s2[k]), Fraction(float(mx[k])))
        assert _is_rounded_sqrt(float(s1[k]), Fraction(float(s2[k])))
    # s^4 tracks the maximum within a few ulps
    assert np.allclose(s1.astype(np.float64) ** 4, np.where(mx == 0, 1.0, mx), rtol=1e-6)
