"""CPU check of the selection's error bound. The top-k kernel decides an entry on its approximate
score v only when v is clear of the decision point by more than twice a per-row bound E on
|v - s * 2^-(e+16+F)| (s the float64 dot product of the block means); everything else it decides
on s itself. This test restates, in numpy, the arithmetic that bound covers (the integer digits of
the means, the six kept digit products, the float32 evaluation of v) and the bound itself, and
checks that the bound holds, on random, badly scaled and extreme-digit mean vectors. It shares no
code with the kernels and none with the oracle; a wrong digit weight, a dropped product or a bound
term too small fails it."""
from fractions import Fraction
import math

import numpy as np
import pytest

RNG = np.random.default_rng(2024)
DIGIT_SHIFT = 21           # |x| * 2^-e in [2^21, 2^22)
ZERO_EXP = -1000


def digits(x):
    """exponent e and the signed base-256 digits (d2, d1, d0) of X = rint(x 2^-e), per channel."""
    amax = np.max(np.abs(x))
    if amax == 0.0:
        return ZERO_EXP, np.zeros((3, x.size), dtype=np.int64)
    e = math.frexp(amax)[1] - 1 - DIGIT_SHIFT          # ilogb(amax) - 21
    X = np.rint(np.ldexp(x, -e)).astype(np.int64)
    assert np.all(np.abs(X) <= 1 << 22)
    d0 = ((X & 255) ^ 128) - 128
    X1 = (X - d0) >> 8
    d1 = ((X1 & 255) ^ 128) - 128
    d2 = (X1 - d1) >> 8
    assert np.all(d2 * 65536 + d1 * 256 + d0 == X) and np.all(np.abs(d2) <= 64)
    return e, np.stack([d2, d1, d0])


def norms_up(x):
    """L1 and L2 norms rounded up to float32 (with the kernel's 2^-40 margin)."""
    def up(v):
        f = np.float32(v)
        return float(np.nextafter(f, np.float32(np.inf))) if float(f) < v else float(f)
    l1 = float(np.sum(np.abs(x))) * (1.0 + 2.0 ** -40)
    l2 = math.sqrt(float(np.sum(x * x))) * (1.0 + 2.0 ** -40)
    return up(l1), up(l2)


def approx_score(dq, dk, shift):
    """v in float32: 2^8 p4 + p3 exact in int32, then (float)(.) * 256 + (float)p2 with one
    rounding (an fma), then scaled by 2^shift."""
    p4 = int(np.dot(dk[0], dq[0]))
    p3 = int(np.dot(dk[0], dq[1]) + np.dot(dk[1], dq[0]))
    p2 = int(np.dot(dk[0], dq[2]) + np.dot(dk[1], dq[1]) + np.dot(dk[2], dq[0]))
    m = (p4 << 8) + p3
    assert -(1 << 31) <= m < (1 << 31)
    hi = np.float32(float(np.float32(m)) * 256.0 + float(np.float32(p2)))   # exact in float64, one rounding
    return float(np.ldexp(hi, shift))


def bound(D, e, qn, F, y1max, y2max):
    """The per-row bound E (v units) and the v units per unit of s."""
    to_v = math.ldexp(1.0, -(e + 16 + F))
    ev = D * 8404992.25 * 2.0 ** -16
    if qn[0] > 0:
        ev += qn[0] * math.ldexp(1.0, -(e + 17))
    if y1max > 0:
        ev += y1max * math.ldexp(1.0, -(F + 17))
    bv = (qn[1] * y2max * to_v + ev) * (1.0 + 2.0 ** -10)
    E = (ev + 2.0 ** -22 * bv + D * 2.0 ** -9) * (1.0 + 2.0 ** -10) + 2.0 ** -126
    return E, to_v


def check_rows(qs, ks):
    """max over all (q, k) pairs of |v - s to_v| / E; asserts it is at most 1."""
    D = qs.shape[1]
    kd = [digits(k) for k in ks]
    F = max(e for e, _ in kd)
    kn = [norms_up(k) for k in ks]
    y1 = max(n[0] for n in kn)
    y2 = max(n[1] for n in kn)
    worst = 0.0
    for q in qs:
        e, dq = digits(q)
        E, to_v = bound(D, e, norms_up(q), F, y1, y2)
        for k, (f, dk) in zip(ks, kd):
            v = approx_score(dq, dk, f - F)
            s = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q, k)), Fraction(0))
            err = abs(Fraction(v) - s * Fraction(to_v))
            assert err <= Fraction(E), (float(err), E)
            worst = max(worst, float(err) / E)
    return worst


@pytest.mark.parametrize("D", [64, 128])
def test_bound_holds_on_random_means(D):
    qs = RNG.standard_normal((6, D)) * 0.3
    ks = RNG.standard_normal((10, D)) * 0.3
    worst = check_rows(qs, ks)
    assert worst > 1e-4      # the bound is not vacuous by orders of magnitude


def test_bound_holds_with_badly_scaled_blocks():
    """Key blocks whose scales span 2^-30 .. 2^10 (shifts far below F), channels spanning 2^-20,
    a zero query block and a zero key block."""
    D = 128
    ks = RNG.standard_normal((12, D)) * np.exp2(RNG.uniform(-30, 10, (12, 1)))
    ks[:, :8] *= 2.0 ** -20
    ks[3] = 0.0
    qs = RNG.standard_normal((5, D)) * np.exp2(RNG.uniform(-12, 6, (5, 1)))
    qs[2] = 0.0
    check_rows(qs, ks)


def test_bound_holds_at_extreme_digits():
    """Means whose integer digits sit at the ends of their ranges (d1, d0 = -128 or 127, |X| at
    2^22), where the dropped products are largest."""
    D = 64
    base = 2.0 ** -3
    # X values near 2^22 with low bytes 0x80 / 0x7f patterns
    pattern = np.array([(1 << 22) - 129, -(1 << 22) + 128, (1 << 21) + 0x7F7F, -((1 << 21) + 0x8080)] * (D // 4),
                       dtype=np.float64)
    q = pattern * base * 2.0 ** -22
    k = pattern[::-1].copy() * base * 2.0 ** -22
    check_rows(np.stack([q, -q]), np.stack([k, -k, q]))


def test_dropped_products_term_is_tight():
    """With means whose integers X are exact (no rounding of x to X), the only error left is the
    three dropped digit products (and the float32 evaluation of v). At extreme digits it reaches
    about half of the bound's dropped-products term, so that term (D * 8404992.25 * 2^-16) can be
    neither left out nor much smaller."""
    D = 64
    pattern = np.array([(1 << 22) - 129, -(1 << 22) + 128, (1 << 21) + 0x7F7F, -((1 << 21) + 0x8080)] * (D // 4),
                       dtype=np.float64) * 2.0 ** -25
    k = pattern[::-1].copy()
    e, dq = digits(pattern)
    f, dk = digits(k)
    assert np.all(np.ldexp(pattern, -e) == np.rint(np.ldexp(pattern, -e)))   # X exact
    v = approx_score(dq, dk, 0)
    s = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(pattern, k)), Fraction(0))
    err = float(abs(Fraction(v) - s * Fraction(math.ldexp(1.0, -(e + 16 + f)))))
    drop = D * 8404992.25 * 2.0 ** -16
    assert 0.4 * drop < err <= drop
