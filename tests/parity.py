"""Helpers of the parity tests: tolerance checks against the oracle's magnitude bounds.

The bar: bit-exact for integer and index work; for floating point, element-wise
|y_gpu - y_oracle| <= rtol * M with M the oracle's sum of |terms| (M = 0 means exact);
rtol = 1e-5 for fp32 arithmetic, 1e-2 for bf16 storage or bf16 matrix-core operands.
"""
import numpy as np

RTOL_F32 = 1e-5
RTOL_BF16 = 1e-2


def assert_close(got, want, mag, rtol, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    mag = np.asarray(mag, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite GPU values" % what
    err = np.abs(got - want)
    bound = rtol * mag
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        ratio = np.max(err / np.maximum(mag, 1e-300))
        raise AssertionError("%s: %d of %d elements outside %g*M (worst err/M %.3g) at %s: got %s "
                             "want %s M %s" % (what, int(bad.sum()), bad.size, rtol, ratio,
                                               idx.tolist(), got[tuple(idx[0])],
                                               want[tuple(idx[0])], mag[tuple(idx[0])]))


def worst_ratio(got, want, mag):
    err = np.abs(np.asarray(got, np.float64) - want)
    m = np.asarray(mag, np.float64)
    r = np.where(m > 0, err / np.where(m > 0, m, 1), np.where(err > 0, np.inf, 0))
    return float(r.max()) if r.size else 0.0
