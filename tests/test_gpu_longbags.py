"""Bags longer than a block's share ("DHEN" notes, 2.1 sum pooling), through the C ABI.

A bag of more than 4096 occurrences is pooled in chunks of 4096 spread over the GPU and its
chunk sums added by a fixed pairwise tree, so its rounding depth D (tests/parity.py,
long_bag_depth) grows with log L instead of L.  The checks use that tight bound g_D:
* one bag of 10^6 rows with all-positive values, where a sum taken row after row in one
  lane group drifts by about sqrt(L) u, far outside g_D;
* long bags of assorted lengths (just above the threshold, exactly on chunk edges, two long
  bags in one chunk, and beside short and empty bags) over several tables, fp32, bf16 and
  fp16 tables, rows of one to several 16-byte vectors, int32 and int64 indices;
* a workspace left full of garbage by the caller, and the same call repeated: same bits.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from sparse_embedding_lookup_amd import ctr
from tests.parity import LONG_BAG, LONG_CHUNK, assert_within, pool_eps
from tests.test_gpu_parity import DEV, TORCH_DTYPE, dev, gpu_table, host, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _pool(t, ids, off, B, T, dim, rb, ws=None):
    out = torch.full((B, T, dim), float("nan"), dtype=torch.float32, device=DEV)
    ctr.ctr_embbag_fwd(t, dev(ids), dev(off), B, T, out, T * dim, dim, row_base=dev(rb),
                       workspace=ws)
    return host(out)


def test_one_positive_bag_of_a_million():
    rows, dim = [100_000], 4
    rng = np.random.default_rng(1)
    vals = rng.uniform(0.5, 1.0, size=(rows[0], dim)).astype(np.float32)
    t = torch.from_numpy(vals).to(DEV)
    tab = orc.Table(rows, dim, "f32", 0, data=vals)
    L = 1_000_000
    ids = rng.integers(0, rows[0], size=L)
    off = np.array([0, L], dtype=np.int64)
    say("one positive bag", L)
    got = _pool(t, ids, off, 1, 1, dim, tab.row_base)
    want, mag = orc.embbag_fwd(tab, ids, off, 1)
    used = assert_within(got, want, pool_eps(off, 1, 1, dim, "f32") * mag, "positive 1M bag",
                         mag=mag)
    assert used <= 1.0
    # a one-row-after-another fp32 sum of the same rows (numpy's sequential accumulate)
    # misses by far more than that bound
    serial = np.add.accumulate(vals[ids], axis=0, dtype=np.float32)[-1]
    drift = float(np.abs(serial - want[0, 0]).max() / mag[0, 0].max())
    bound = float(pool_eps(off, 1, 1, dim, "f32").max())
    say("serial drift %.3g, tree bound %.3g" % (drift, bound))
    assert drift > 4 * bound, (drift, bound)


def _mixed_csr(rng, T, B, rows):
    """Lengths: mostly short, some empty, and long bags at chosen places: just above the
    threshold, on chunk edges, and two long bags sharing a chunk."""
    lens = rng.integers(0, 40, size=(T, B))
    lens[rng.random((T, B)) < 0.1] = 0
    longs = [LONG_BAG + 1, LONG_CHUNK * 3, 50_000, 2 * LONG_CHUNK + 5, LONG_BAG + 1, 9_000]
    spots = [(0, 3), (0, 4), (1, 0), (T - 1, B - 1), (1, B // 2), (1, B // 2 + 1)]
    for (t, b), L in zip(spots, longs):
        lens[t, b] = L
    # make one long bag start exactly on a chunk edge: pad the bag before it
    flat = lens.reshape(-1)
    pos = spots[2][0] * B + spots[2][1]
    start = int(flat[:pos].sum())
    flat[pos - 1] += (-start) % LONG_CHUNK
    off = np.zeros(T * B + 1, dtype=np.int64)
    off[1:] = np.cumsum(flat)
    assert off[pos] % LONG_CHUNK == 0
    ids = np.concatenate([rng.integers(0, rows[t], size=int(lens[t].sum())) for t in range(T)])
    return ids, off


@pytest.mark.parametrize("dtype,dim", [("f32", 4), ("f32", 64), ("bf16", 128), ("f16", 32),
                                       ("f32", 512), ("bf16", 1024)])
@pytest.mark.parametrize("itype", ["i64", "i32"])
def test_long_bags_among_short_ones(dtype, dim, itype):
    rng = np.random.default_rng(dim + (7 if itype == "i32" else 0))
    T, B = 3, 97
    rows = [20_000, 3_000, 50_000]
    ids, off = _mixed_csr(rng, T, B, rows)
    ids = ids.astype(np.int32 if itype == "i32" else np.int64)
    say("long bags", dtype, dim, itype, ids.size)
    t = gpu_table(rows, dim, dtype, 5)
    tab = orc.Table(rows, dim, dtype, 5)
    got = _pool(t, ids, off, B, T, dim, tab.row_base)
    want, mag = orc.embbag_fwd(tab, ids, off, B)
    assert_within(got, want, pool_eps(off, B, T, dim, dtype) * mag, "long bags " + dtype,
                  mag=mag)
    lens = np.diff(off).reshape(T, B).T
    np.testing.assert_array_equal(got[lens == 0], 0.0)


def test_garbage_workspace_and_repeat_give_the_same_bits():
    rng = np.random.default_rng(3)
    T, B, dim = 3, 97, 32
    rows = [20_000, 3_000, 50_000]
    ids, off = _mixed_csr(rng, T, B, rows)
    t = gpu_table(rows, dim, "bf16", 9)
    rb = orc.Table(rows, dim, "bf16", 9).row_base
    nb = ctr.embbag_fwd_workspace_bytes(ids.size, dim)
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device=DEV)
    a = _pool(t, ids, off, B, T, dim, rb, ws)
    b = _pool(t, ids, off, B, T, dim, rb, ws)
    c = _pool(t, ids, off, B, T, dim, rb, torch.zeros(nb, dtype=torch.uint8, device=DEV))
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)


def test_tensor_dtype_map_covers_tables():
    assert set(TORCH_DTYPE) == {"f32", "bf16", "f16"}
