"""Inference-side lookup from an exported sparse-embedding dictionary on the GPU ("How
TensorNet Supercharges Sparse Feature Training on TensorFlow", "Inference Optimization"),
with the hot-row HBM cache of a hierarchical parameter server, through the C ABI.

* Lookup values are integers: bit-exact against the oracle's sorted search, for a
  half-full table and for a table filled to capacity - 1 (long probe runs).
* Repeated and negative keys are counted in the status words.
* Pooled lookups match the oracle within rtol * M.  The full table in HBM, in pinned host
  memory (read over the host link), or with no cache at all gives the same bits: the cache
  holds copies, and the sum order is the occurrence order either way.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from sparse_embedding_lookup_amd import ctr, workloads
from tests.parity import assert_within, pool_eps
from tests.test_gpu_parity import DEV, dev, host, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _dictionary(n, key_hi, seed):
    rng = np.random.default_rng(seed)
    keys = rng.choice(key_hi, size=n, replace=False).astype(np.int64)
    rows = rng.permutation(n).astype(np.int32)
    hot = np.where(rng.random(n) < 0.25, rng.integers(0, 5000, n), -1).astype(np.int32)
    return rng, keys, rows, hot


@pytest.mark.parametrize("n,cap", [(100_000, None), (4095, 4096), (1, 2)])
def test_dict_lookup_bit_exact(n, cap):
    say("dict lookup", n, cap)
    rng, keys, rows, hot = _dictionary(n, 10 ** 11, n)
    cap = cap or ctr.dict_capacity(n)
    slots, status = ctr.ctr_dict_build(dev(keys), dev(rows), dev(hot), cap)
    np.testing.assert_array_equal(host(status), [0, 0, 0])
    m = 3 * n + 1000
    ids = np.concatenate([rng.choice(keys, size=m // 2), rng.integers(0, 10 ** 11, m // 2),
                          np.array([-1, 0, 2 ** 63 - 1])]).astype(np.int64)
    got = host(ctr.ctr_dict_lookup(dev(ids), slots, cap))[:ids.size]
    np.testing.assert_array_equal(got, orc.dict_lookup(keys, rows, hot, ids))


def test_dict_repeated_and_negative_keys():
    rng, keys, rows, hot = _dictionary(5000, 10 ** 9, 3)
    keys[10:20] = keys[0]                          # 10 repeats of one key
    keys[30:33] = [-1, -7, -(2 ** 62)]
    cap = ctr.dict_capacity(keys.size)
    slots, status = ctr.ctr_dict_build(dev(keys), dev(rows), dev(hot), cap)
    np.testing.assert_array_equal(host(status), [10, 3, 0])
    v = int(host(ctr.ctr_dict_lookup(dev(keys[:1]), slots, cap))[0])
    allowed = {(int(h) + 1) << 32 | int(r) for k, r, h in zip(keys, rows, hot) if k == keys[0]}
    assert v in allowed
    ok = np.ones(keys.size, bool)
    ok[10:20] = False
    ok[0] = False
    ok[30:33] = False
    got = host(ctr.ctr_dict_lookup(dev(keys[ok]), slots, cap))[:int(ok.sum())]
    want = ((hot[ok].astype(np.int64) + 1) << 32) | rows[ok].astype(np.int64)
    np.testing.assert_array_equal(got, want)
    neg = host(ctr.ctr_dict_lookup(dev(keys[30:33]), slots, cap))[:3]
    np.testing.assert_array_equal(neg, [-1, -1, -1])


def _pool_setup(dtype, dim, seed=11):
    w = workloads.dictionary(seed=seed, batch=512, slots=100, entries=200_000, hot=20_000)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    table = torch.empty((w.entries, dim), dtype=tdt, device=DEV)
    ctr.ctr_init_tables_hash(table, [w.entries], w.table_seed)
    # the cache holds copies of the rows of the H most popular IDs, slot = rank - 1
    hot_rows = table[dev(w.dict_rows[:w.hot].astype(np.int64))].contiguous()
    slots, status = ctr.ctr_dict_build(dev(w.dict_keys), dev(w.dict_rows), dev(w.hot_slots),
                                       ctr.dict_capacity(w.entries))
    np.testing.assert_array_equal(host(status), [0, 0, 0])
    values = ctr.ctr_dict_lookup(dev(w.indices), slots, ctr.dict_capacity(w.entries))
    return w, table, hot_rows, values


@pytest.mark.parametrize("dtype,dim", [("f32", 32), ("bf16", 64), ("f32", 256)])
def test_dict_pool_matches_oracle_and_tiers_agree(dtype, dim):
    say("dict pool", dtype, dim)
    w, table, hot_rows, values = _pool_setup(dtype, dim)
    B, S = w.batch, w.slots
    n = w.nnz
    offsets = dev(w.offsets)

    def pool(hot, tab):
        out = torch.full((n, dim), float("nan"), device=DEV)
        ctr.ctr_dict_embbag_fwd(values, n, offsets, n, 1, hot, tab, out, dim, 0)
        return host(out)

    got = pool(hot_rows, table)
    vals = host(values)[:n]
    hits = float(np.mean(vals >= 0))
    cached = float(np.mean((vals >= 0) & ((vals >> 32) > 0)))
    say("hit rate %.4f, cache hit rate %.4f" % (hits, cached))
    assert 0.5 < hits < 1.0 and 0.3 < cached < hits   # both tiers and misses are exercised
    tab = orc.Table([w.entries], dim, dtype, w.table_seed)
    want, mag = orc.dict_pool(tab, orc.dict_lookup(w.dict_keys, w.dict_rows, w.hot_slots,
                                                   w.indices), w.offsets, n, 1)
    assert_within(got, want.reshape(n, dim),
                  pool_eps(w.offsets, n, 1)[:, 0, :] * mag.reshape(n, dim), "dict pool",
                  mag=mag.reshape(n, dim))
    # the same bits with no cache, and with the table in pinned host memory
    np.testing.assert_array_equal(pool(None, table), got)
    host_table = torch.empty(table.shape, dtype=table.dtype, pin_memory=True)
    host_table.copy_(table)
    np.testing.assert_array_equal(pool(hot_rows, host_table), got)


def test_dict_pool_bags_across_tables():
    # bags of several IDs over two "tables" (bag (t, b) at t * batch + b), empty bags included
    w, table, hot_rows, values = _pool_setup("f32", 32, seed=12)
    rng = np.random.default_rng(4)
    T, B = 2, 300
    lengths = rng.integers(0, 7, size=T * B)
    off = np.zeros(T * B + 1, dtype=np.int64)
    off[1:] = np.cumsum(lengths)
    n = int(off[-1])
    assert n <= w.nnz
    out = torch.full((B, T, 32), float("nan"), device=DEV)
    ctr.ctr_dict_embbag_fwd(values, n, dev(off), B, T, hot_rows, table, out, T * 32, 32)
    vals = orc.dict_lookup(w.dict_keys, w.dict_rows, w.hot_slots, w.indices[:n])
    want, mag = orc.dict_pool(orc.Table([w.entries], 32, "f32", w.table_seed), vals, off, B, T)
    assert_within(host(out), want, pool_eps(off, B, T) * mag, "dict pool bags", mag=mag)
