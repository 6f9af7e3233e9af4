"""Pins of the oracle's stochastic rounding ("DHEN" notes, 6.4 "Common Optimizations":
low-precision embeddings updated with stochastic rounding) against facts that do not come
from the oracle itself.

* The bracketing values come from binary32 bit patterns (truncating the low 16 bits, and the
  next bf16 pattern away from zero), a different route from the oracle's frexp arithmetic.
* Over all 2^16 random integers, exactly `low16` round away from zero.  So the mean of
  SR(x) over r is x itself, and a wrong comparison (<= for <), a wrong quantum or a sign
  slip changes the count.
* Special values, subnormals and the overflow to infinity follow IEEE-754 bfloat16.
* The random bits are uniform (chi-square); each group of four columns takes the four
  16-bit fields of one splitmix64 output (a pinned generator).
* The drift test: repeated updates far below half an ulp.  Nearest-even never moves the
  value; the stochastic mean follows the exact sum.
No GPU is used.
"""
import numpy as np
import pytest

from oracle import oracle as orc

from sparse_embedding_lookup_amd import ctr


def _bits(x: float) -> int:
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])


def _f(b: int) -> float:
    return float(np.array([b & 0xFFFFFFFF], dtype=np.uint32).view(np.float32)[0])


def _neighbours(x: float):
    """(lo, hi): x's bf16 truncation toward zero and the next bf16 away from zero, from the
    binary32 pattern (sign-magnitude: the next magnitude is the next pattern)."""
    b = _bits(x)
    lo = b & 0xFFFF0000
    return _f(lo), _f(lo + 0x10000)


CASES = [1.0 + 2 ** -9, -(1.0 + 2 ** -9), 1.0 + 3 * 2 ** -10, 0.1, -0.3333333,
         3.0e-39, -1.0e-40,                    # binary32 subnormals (bf16 subnormal range)
         1.17549435e-38,                       # smallest normal binary32
         np.float32(2.0) - np.float32(2 ** -23),   # just below a binade edge
         -65504.0 * 1.0001, 1.2345e30]


@pytest.mark.parametrize("x", CASES)
def test_sr_exhaustive_count_is_low16(x):
    x = float(np.float32(x))
    low = _bits(x) & 0xFFFF
    lo, hi = _neighbours(x)
    out = np.array([orc.sr_bf16(x, r) for r in range(1 << 16)])
    assert set(np.unique(out)) <= {lo, hi}
    ups = int(np.count_nonzero(out == hi)) if hi != lo else 0
    assert ups == low
    # the mean over r is x exactly (lo + (hi - lo) * low / 2^16 is x's binary32 value)
    assert lo + (hi - lo) * ups / 65536.0 == x


def test_sr_decision_is_r_below_low_half():
    x = float(np.float32(1.0 + 2 ** -9))       # low 16 bits = 0x4000
    lo, hi = _neighbours(x)
    assert orc.sr_bf16(x, 0x3FFF) == hi
    assert orc.sr_bf16(x, 0x4000) == lo
    assert orc.sr_bf16(-x, 0) == -hi           # away from zero for negatives


def test_sr_special_values():
    for v in [0.0, -0.0, 1.0, -2.5, 1.5, float("inf"), float("-inf")]:
        for r in (0, 1, 0x7FFF, 0xFFFF):
            assert orc.sr_bf16(v, r) == v      # exact bf16 values never move
    assert np.isnan(orc.sr_bf16(float("nan"), 5))
    big = _f(0x7F7FFFFF)                       # largest binary32: above the largest bf16
    assert orc.sr_bf16(big, 0) == float("inf")
    assert orc.sr_bf16(big, 0xFFFF) == _f(0x7F7F0000)


def test_sr_bits_uniform_and_splitmix():
    seed, dim = 0x1234_5678_9ABC_DEF0, 128
    n = 1 << 15
    rs = np.array([orc.sr_bits(seed, k // dim, k % dim, dim) for k in range(n)])
    assert rs.min() >= 0 and rs.max() < (1 << 16)
    counts = np.bincount(rs >> 8, minlength=256)
    chi2 = float(((counts - n / 256) ** 2 / (n / 256)).sum())
    assert chi2 < 255 + 6 * np.sqrt(2 * 255)   # about a 1e-6 false-alarm level
    # one output of the pinned generator per four columns, from state seed ^ (key*dim + c4);
    # column c4 + e takes its 16-bit field e
    for key, c4 in [(0, 0), (7, 4), (123456, 124)]:
        z = orc.splitmix64_stream(seed ^ (key * dim + c4), 1)[0]
        for e in range(4):
            assert orc.sr_bits(seed, key, c4 + e, dim) == (z >> (16 * e)) & 0xFFFF


def test_sgd_sr_drift_follows_exact_sum():
    # 256 bf16 values 1.0, each updated 64 times with lr*g = 2^-12 (ulp(1) = 2^-7 above,
    # 2^-8 below): nearest-even rounds every update away, stochastic rounding's mean
    # follows 1 - 64 * 2^-12 = 0.984375
    rows, dim, steps = 64, 4, 64
    tab = orc.Table([rows], dim, "bf16", 3, data=np.ones((rows, dim), np.float32))
    uniq = np.arange(rows)
    g = np.full((rows, dim), 2.0 ** -12, np.float32)
    cur = np.ones((rows, dim))
    near = np.ones((rows, dim))
    for k in range(steps):
        t = orc.Table([rows], dim, "bf16", 3, data=cur.astype(np.float32))
        cur = orc.sparse_sgd_sr(t, uniq, g, 1.0, 1000 + k)
        tn = orc.Table([rows], dim, "bf16", 3, data=near.astype(np.float32))
        near, _ = orc.sparse_sgd(tn, uniq, g.astype(np.float64), g.astype(np.float64), 1.0)
    assert np.all(near == 1.0)
    exact = 1.0 - steps * 2.0 ** -12
    # each update moves by at most one ulp (2^-8 below 1); the 256 trajectories are
    # independent, so the mean is within a few standard errors of the exact value
    assert abs(cur.mean() - exact) < 6 * 2.0 ** -8 * np.sqrt(steps) / np.sqrt(rows * dim)
    assert cur.max() <= 1.0 and cur.min() >= 1.0 - steps * 2.0 ** -8


def test_sgd_sr_lr0_keeps_stored_values_and_brackets():
    tab = orc.Table([50, 70], 16, "bf16", 11)
    uniq = np.array([0, 5, 49, 50, 119])
    g = np.random.default_rng(0).standard_normal((5, 16)).astype(np.float32)
    stored = orc.gather_rows(tab, uniq)
    same = orc.sparse_sgd_sr(tab, uniq, g, 0.0, 42)
    np.testing.assert_array_equal(same, stored)
    new = orc.sparse_sgd_sr(tab, uniq, g, 0.25, 42)
    # the binary32 fused multiply-add: the exact value (here exact in float64) rounded once
    x = (stored - 0.25 * g.astype(np.float64)).astype(np.float32)
    for v, xv in zip(new.ravel(), x.ravel()):
        lo, hi = _neighbours(float(xv))
        assert v in (lo, hi)


def test_step_seed_is_splitmix_stream():
    # ctr_sr_step_seed is host code of the library (no GPU): output k of the splitmix64
    # stream started at base, checked against the oracle's pinned generator
    for base in (0, 0x5EED_0000_5EED_0005, 2 ** 64 - 1):
        want = orc.splitmix64_stream(base, 5)
        assert [ctr.ctr_sr_step_seed(base, k) for k in range(5)] == want
