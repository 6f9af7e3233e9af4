"""Pins of the oracle's binary16 storage ("DHEN" notes, 6.4 "Common Optimizations": FP16
embeddings, updated with stochastic rounding) against facts that do not come from the oracle.

* Nearest-even rounding to binary16 equals numpy's float64 -> float16 conversion (a
  correctly rounded library routine) on random values of every binade, on every tie between
  neighbouring binary16 values, through the subnormal range and at the overflow threshold.
* Stochastic rounding brackets x between binary16 neighbours taken from numpy (the float16
  truncation and np.nextafter away from zero), and over all 2^16 random integers exactly
  ceil(2^16 p) round away from zero, p = (|x| - |lo|) / q computed with exact rationals.  In
  the normal range p is a multiple of 2^-13, so the count is 8 times the 13 dropped fraction
  bits and the mean of SR(x) is x itself.
* Special values and the overflow to infinity follow IEEE-754 binary16.
* The SGD update of a binary16 table rounds the exact w - lr g once (numpy, from exactly
  representable inputs); its stochastic form is the same SR of the binary32 fused
  multiply-add, element by element.
No GPU is used.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as orc


def _f16(x: float) -> float:
    with np.errstate(over="ignore"):
        return float(np.float16(x))


def test_round_f16_matches_numpy_random():
    rng = np.random.default_rng(1)
    # every binade from deep below the subnormals to beyond the largest finite value
    e = rng.uniform(-30, 17.2, size=20000)
    x = np.sign(rng.standard_normal(e.size)) * 2.0 ** e
    for v in x:
        assert orc.round_f16(float(v)) == _f16(float(v)), v


def test_round_f16_ties_go_to_even():
    # all positive finite binary16 values a < b: the midpoint is exact in binary64
    vals = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2.0
    for lo, hi, m in zip(vals[:-1], vals[1:], mids):
        want = lo if (np.float16(lo).view(np.uint16) & 1) == 0 else hi
        assert orc.round_f16(m) == want
        assert orc.round_f16(-m) == -want
        assert orc.round_f16(m) == _f16(m)


def test_round_f16_overflow_and_specials():
    assert orc.round_f16(65504.0) == 65504.0
    assert orc.round_f16(65519.99) == 65504.0
    assert orc.round_f16(65520.0) == math.inf          # the tie goes to the even 2^16
    assert orc.round_f16(-65520.0) == -math.inf
    assert orc.round_f16(1e30) == math.inf
    assert orc.round_f16(math.inf) == math.inf
    assert math.isnan(orc.round_f16(math.nan))
    assert orc.round_f16(0.0) == 0.0 and math.copysign(1.0, orc.round_f16(-0.0)) == -1.0
    assert orc.round_f16(2.0 ** -25) == 0.0            # tie between 0 and the least subnormal
    assert orc.round_f16(2.0 ** -25 * 1.0001) == 2.0 ** -24
    assert orc.round_f16(3 * 2.0 ** -25) == 2.0 ** -23  # tie 1.5 q -> 2 q (even)
    assert orc.round_f16(2.0 ** -14 - 2.0 ** -26) == 2.0 ** -14   # subnormal to normal


def _bracket(x: float):
    """(lo, hi): x truncated toward zero to binary16 and the next binary16 away from zero,
    from numpy's float16 grid."""
    with np.errstate(over="ignore"):
        r = np.float16(x)                               # nearest
        if abs(float(r)) > abs(x):
            r = np.nextafter(r, np.float16(0.0))
        lo = float(r)
        hi = float(np.nextafter(r, np.float16(math.copysign(np.inf, x))))
    return lo, hi


X_CASES = [1.0 + 2.0 ** -20, 1.0 + 2.0 ** -11 + 2.0 ** -23, 3.14159265, -2.71828183, 1e-3,
           -6.1e-5, 6.0e-8, 3.0e-8, 1.7e-6, 65500.0, -12345.678, 0.1, 2.0 ** -14 - 2.0 ** -30,
           1e-40, 65519.0, 65535.5]


@pytest.mark.parametrize("x", X_CASES)
def test_sr_f16_exhaustive_count(x):
    x = float(np.float32(x))                            # the kernels round binary32 values
    lo, hi = _bracket(x)
    q = Fraction(abs(hi) - abs(lo)) if math.isfinite(hi) else Fraction(32)
    p = (abs(Fraction(x)) - abs(Fraction(lo))) / q
    want_up = math.ceil(p * 65536)
    outs = np.array([orc.sr_f16(x, r) for r in range(65536)])
    hi_v = hi if abs(hi) <= 65504.0 else math.copysign(math.inf, x)
    assert set(np.unique(outs)) <= {lo, hi_v}
    up = int(np.sum(outs == hi_v)) if hi_v != lo else 0
    assert up == want_up
    # the decision is r < threshold: the first want_up integers go up
    assert np.all(outs[:want_up] == hi_v) and np.all(outs[want_up:] == lo)
    if abs(x) >= 2.0 ** -14 and abs(x) < 65504.0:
        assert want_up == 8 * (int(np.float32(abs(x)).view(np.uint32)) & 0x1FFF)
        mean = Fraction(lo) + Fraction(hi - lo) * Fraction(up, 65536)
        assert mean == Fraction(x)                      # unbiased exactly


def test_sr_f16_specials_and_exact_values():
    for r in (0, 1, 0x7FFF, 0xFFFF):
        for v in (0.0, 1.0, -2.0, 65504.0, 2.0 ** -24, -(2.0 ** -14), 0.5 + 2.0 ** -11):
            assert orc.sr_f16(v, r) == v
        assert orc.sr_f16(math.inf, r) == math.inf
        assert orc.sr_f16(-math.inf, r) == -math.inf
        assert math.isnan(orc.sr_f16(math.nan, r))
        assert orc.sr_f16(65536.0, r) == math.inf
        assert orc.sr_f16(-1e6, r) == -math.inf
    assert math.copysign(1.0, orc.sr_f16(-0.0, 5)) == -1.0


def test_sparse_sgd_f16_closed_form():
    rows, dim = [300, 200], 8
    tab = orc.Table(rows, dim, "f16", 91)
    rng = np.random.default_rng(3)
    uniq = np.sort(rng.choice(500, size=120, replace=False)).astype(np.int64)
    g = rng.standard_normal((uniq.size, dim)).astype(np.float32)
    lr = 2.0 ** -7                                      # w - lr g exact in binary64
    new, nmag = orc.sparse_sgd(tab, uniq, g.astype(np.float64), np.abs(g).astype(np.float64),
                               lr)
    w = orc.gather_rows(tab, uniq).astype(np.float64)
    exact = w - lr * g.astype(np.float64)
    np.testing.assert_array_equal(new, exact.astype(np.float16).astype(np.float64))
    np.testing.assert_array_equal(nmag, np.abs(w) + lr * np.abs(g))
    # the table holds binary16 values
    np.testing.assert_array_equal(w, w.astype(np.float16).astype(np.float64))


def test_sparse_sgd_sr_f16_elementwise():
    rows, dim = [100], 8
    tab = orc.Table(rows, dim, "f16", 17)
    rng = np.random.default_rng(4)
    uniq = np.array([3, 50, 99], dtype=np.int64)
    g = (rng.standard_normal((3, dim)) * 1e-3).astype(np.float32)
    seed, lr = 0xABCDEF, 0.5
    got = orc.sparse_sgd_sr(tab, uniq, g, lr, seed)
    w = orc.gather_rows(tab, uniq).astype(np.float32)
    for u in range(3):
        for c in range(dim):
            x = float(np.float32(np.float64(w[u, c]) - np.float64(np.float32(lr) * g[u, c])))
            # fmaf(-lr, g, w) in binary32: the product lr * g is exact here (lr = 2^-1)
            want = orc.sr_f16(x, orc.sr_bits(seed, int(uniq[u]), c, dim))
            assert got[u, c] == want
            lo, hi = _bracket(x)
            assert got[u, c] in (lo, hi)
