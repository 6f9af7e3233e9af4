"""Pins of the oracle's dictionary lookup and pooled lookup ("How TensorNet Supercharges
Sparse Feature Training on TensorFlow", "Inference Optimization": online inference reads a
pre-exported sparse embedding dictionary keyed by raw ID), against brute force that shares
nothing with the oracle's sorted search: a Python dict, and direct numpy sums.  The
workload's ID bijection is checked against its definition in exact integer arithmetic.
No GPU is used.
"""
import numpy as np

from oracle import oracle as orc
from sparse_embedding_lookup_amd import workloads


def _random_dictionary(rng, n, key_hi):
    keys = rng.choice(key_hi, size=n, replace=False).astype(np.int64)
    rows = rng.permutation(n).astype(np.int32)
    hot = np.where(rng.random(n) < 0.3, rng.integers(0, 1000, n), -1).astype(np.int32)
    return keys, rows, hot


def test_lookup_matches_python_dict():
    rng = np.random.default_rng(0)
    keys, rows, hot = _random_dictionary(rng, 2000, 10 ** 6)
    keys[0], keys[1] = 0, 2 ** 62                  # the extremes of the key range
    d = {int(k): (int(h) + 1) << 32 | int(r) for k, r, h in zip(keys, rows, hot)}
    ids = np.concatenate([rng.choice(keys, 3000), rng.integers(0, 10 ** 6, 3000),
                          np.array([-1, -5, 0, 2 ** 62, 2 ** 63 - 1])]).astype(np.int64)
    got = orc.dict_lookup(keys, rows, hot, ids)
    want = np.array([d.get(int(x), -1) if x >= 0 else -1 for x in ids], dtype=np.int64)
    np.testing.assert_array_equal(got, want)
    # without a cache, the high half is zero
    got0 = orc.dict_lookup(keys, rows, None, ids[:100])
    want0 = np.array([int(rows[np.nonzero(keys == x)[0][0]]) if x in d else -1
                      for x in ids[:100]], dtype=np.int64)
    np.testing.assert_array_equal(got0, want0)


def test_pool_matches_direct_sums():
    rng = np.random.default_rng(1)
    N, d, B, T = 300, 8, 40, 2
    W = rng.standard_normal((N, d)).astype(np.float32)
    tab = orc.Table([N], d, "f32", 5, data=W)
    lengths = rng.integers(0, 6, size=T * B)
    off = np.zeros(T * B + 1, dtype=np.int64)
    off[1:] = np.cumsum(lengths)
    n = int(off[-1])
    rows = rng.integers(0, N, n)
    hs = rng.integers(0, 3, n)                     # cache slot + 1 (0: not cached)
    values = np.where(rng.random(n) < 0.2, -1, (hs << 32) | rows).astype(np.int64)
    out, mag = orc.dict_pool(tab, values, off, B, T)
    want = np.zeros((B, T, d))
    for s in range(T * B):
        t, b = divmod(s, B)
        for k in range(off[s], off[s + 1]):
            if values[k] >= 0:
                want[b, t] += W[values[k] & 0xFFFFFFFF].astype(np.float64)
    np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-13)
    assert np.all(mag >= np.abs(out) - 1e-12)
    empty = (lengths == 0).reshape(T, B).T
    assert np.all(out[empty] == 0.0)


def test_workload_keys_are_the_rank_bijection():
    K = 10 ** 11
    r = np.random.default_rng(2).integers(1, K + 1, 50_000)
    fast = workloads._affine_keys(r, K)
    exact = np.array([((int(x) - 1) * 38_196_601_123 + 12_345_678_901) % K + 1 for x in r])
    np.testing.assert_array_equal(fast, exact)
    w = workloads.dictionary(batch=64, slots=10, entries=100_000, hot=1000)
    assert np.unique(w.dict_keys).size == w.entries            # distinct dictionary IDs
    assert w.dict_keys.min() >= 1 and w.dict_keys.max() <= K
    assert np.array_equal(np.sort(w.dict_rows), np.arange(w.entries))
    assert np.all(w.hot_slots[:1000] == np.arange(1000)) and np.all(w.hot_slots[1000:] == -1)
