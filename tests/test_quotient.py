"""Host check of the division used by the GPU quantizers (CPU only).

The kernels compute f32(x / s) as q0 = f32(x * r), e = fma(-q0, s, x),
q = fma(e, r, q0) with r = f32(1 / s) -- one Markstein correction (Muller et
al., Handbook of Floating-Point Arithmetic, "Newton-Raphson-based division").
The codes must equal the oracle's, which divides in IEEE f32, so the
quotient must be the correctly rounded one wherever it can decide a code:
here it is emulated with exact rational arithmetic and compared with
numpy's IEEE division on random pairs and on exact half-way cases."""
from fractions import Fraction

import numpy as np
import pytest


def _round_f32(v):
    """Nearest float32 to the rational v, ties to even (normal range)."""
    if v == 0:
        return np.float32(0.0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # scale so that 2^23 <= m < 2^24
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    scaled = a / Fraction(2) ** (e - 23)
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return np.float32(sign * float(Fraction(m) * Fraction(2) ** (e - 23)))


def _fma(a, b, c):
    return _round_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def _quotient(x, s):
    x, s = np.float32(x), np.float32(s)
    r = np.float32(1.0) / s
    q0 = np.float32(x * r)
    e = _fma(-q0, s, x)
    return _fma(e, r, q0)


def test_round_f32_matches_numpy_casts():
    rng = np.random.default_rng(0)
    for v in rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 6, 2000):
        assert _round_f32(Fraction(float(v))) == np.float32(v)


def test_random_pairs_give_the_ieee_quotient():
    rng = np.random.default_rng(1)
    n = 20000
    x = (rng.standard_normal(n) * 10.0 ** rng.integers(-4, 4, n)).astype(np.float32)
    amax = np.abs(x) * (1.0 + rng.random(n) * 3.0)
    for qmax in (127.0, 448.0):
        s = (amax / qmax).astype(np.float32)
        for xi, si in zip(x, s):
            q = np.float32(xi) / np.float32(si)
            if abs(q) >= 2.0 ** -20:
                assert _quotient(xi, si) == q, (xi, si)


@pytest.mark.parametrize("scale", [1.0, 3.0, 0.75, 0.125, 5.0, 1.0 / 3.0])
def test_half_way_quotients(scale):
    """value = (k + 1/2) * s exactly: the quotient is a tie of the int8 rounding,
    and a one-ulp error would flip the code."""
    s = np.float32(scale)
    for k in range(-127, 127):
        x = np.float32((k + 0.5) * float(s))
        if Fraction(float(x)) != Fraction(k) * Fraction(float(s)) + Fraction(float(s)) / 2:
            continue  # not exact in f32 for this scale
        assert _quotient(x, s) == np.float32(x) / s == np.float32(k + 0.5)


def test_the_correction_is_needed():
    """Without the correction step (q0 = f32(x * r) alone) the quotient is off
    by an ulp for a good share of pairs: the check above has teeth."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal(2000).astype(np.float32)
    s = (np.abs(rng.standard_normal(2000)) / 127.0).astype(np.float32)
    q0 = x * (np.float32(1.0) / s)
    assert np.mean(q0 != x / s) > 0.05
