"""The batched router accepts an FP64 sum of FP16 products as exact when the
sum of the products' magnitudes is below 31: every FP16 value is an integer
multiple of 2^-24, so every product and every partial sum is one of 2^-48, and
below 2^5 = 2^53 * 2^-48 each is representable in FP64, so no addition rounds.
Checked here against exact rational arithmetic, in several summation orders,
with FP16 values down to subnormals; and a case just above the bound where the
FP64 sum does round."""
from fractions import Fraction

import numpy as np


def _fp16(rng, n, scale):
    v = (rng.standard_normal(n) * scale).astype(np.float16)
    v[rng.integers(0, n, n // 16)] = np.float16(2.0 ** -24) * rng.integers(-1023, 1024, n // 16)
    return v


def _sum64(p, order):
    s = 0.0
    for i in order:
        s += float(p[i])
    return s


def test_fp64_sum_is_exact_below_the_bound():
    rng = np.random.default_rng(5)
    checked = 0
    for trial in range(40):
        n = 2048
        x = _fp16(rng, n, 1.0)
        w = _fp16(rng, n, 0.02)
        p = x.astype(np.float64) * w.astype(np.float64)  # exact: 22 significant bits
        S = float(np.sum(np.abs(p)))
        if S >= 31.0:
            continue
        exact = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, w)), Fraction(0))
        for order in (range(n), range(n - 1, -1, -1), rng.permutation(n)):
            assert Fraction(_sum64(p, order)) == exact
        checked += 1
    assert checked >= 20


def test_fp64_sum_can_round_above_the_bound():
    # 2^5 + 2^-48 needs 54 significant bits: the FP64 sum of these products
    # rounds, so no bound above 2^5 could be used
    a = np.array([2.0 ** 5, 2.0 ** -48])
    assert Fraction(float(a[0]) + float(a[1])) != Fraction(2 ** 5) + Fraction(1, 2 ** 48)
    # the products are FP16 x FP16: 2^5 = 2^3 * 2^2 and 2^-48 = 2^-24 * 2^-24
    assert float(np.float16(2.0 ** 3)) * float(np.float16(2.0 ** 2)) == 2.0 ** 5
    assert float(np.float16(2.0 ** -24)) ** 2 == 2.0 ** -48
