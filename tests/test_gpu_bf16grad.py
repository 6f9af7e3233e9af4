"""The bf16 gradient of a bf16 interaction: the MFMA backward stores dZ rounded to bf16, and
the pooling's backward reads bf16 gradient rows and sums them in fp32.

* The bf16 dZ is exactly the fp32 dZ of the same kernel rounded to nearest-even: same
  arithmetic, only the store differs.
* Row sums from bf16 gradients equal the row sums of the same values widened to fp32, bit
  for bit, when the values are small integers.  Their fp32 sums are exact in any order, and
  the two dtypes use different slot depths.  This holds for row gradients only, with the
  nearest-even update, and with stochastic rounding.  For random values the bf16 path
  matches the oracle within rtol * M.
* Every row width of the first level's lanes (8 columns per lane for widths that are a
  multiple of 8 up to 512: 1 to 64 lanes per row; 4 columns otherwise), with bf16, fp32 and
  binary16 tables: integer-valued rows give the fp32 path's bits for the row sums and for the
  updated table (both roundings), and random rows match the oracle within the tree's bound.
* A Criteo-shaped step with a bf16 dZ stays within the chained tolerance of the oracle.
  That is test_end_to_end_dlrm_step, since FrontEnd keeps dZ in bf16 when the interaction
  computes in bf16.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from sparse_embedding_lookup_amd import ctr, workloads
from tests.parity import assert_close, gamma, segreduce_depth
from tests.test_gpu_parity import DEV, dev, gpu_table, host, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("B,F,d", [(100, 27, 128), (67, 65, 128), (40, 5, 16), (13, 100, 64)])
def test_interaction_bwd_bf16_out_is_rounded_fp32(B, F, d):
    say("interaction bwd bf16 out", B, F, d)
    rng = np.random.default_rng(F)
    Z = dev(rng.standard_normal((B, F, d)).astype(np.float32))
    dR = dev(rng.standard_normal((B, d + F * (F - 1) // 2)).astype(np.float32))
    d32 = ctr.ctr_dot_interaction_bwd(Z, dR, ctr.CTR_BF16)
    d16 = ctr.ctr_dot_interaction_bwd(Z, dR, ctr.CTR_BF16,
                                      torch.empty(Z.shape, dtype=torch.bfloat16, device=DEV))
    assert torch.equal(d16, d32.to(torch.bfloat16))


def _bags_and_unique(name):
    w = {"criteo_b256": lambda: workloads.criteo(batch=256),
         "large_t4_b256": lambda: workloads.large(batch=256, tables=4, rows=20_000)}[name]()
    keys = orc.form_keys(w.indices, w.offsets, w.num_tables, w.batch, w.row_base)
    uniq, inv, perm, seg = orc.unique(keys)
    bag_of = np.searchsorted(w.offsets, np.arange(w.nnz), side="right") - 1
    quads = np.zeros((w.nnz, 4), dtype=np.int32)
    quads[:, 0], quads[:, 1] = inv[perm], bag_of[perm]
    quads[:, 2:] = uniq[inv[perm]].astype(np.int64).view(np.int32).reshape(-1, 2)
    return w, uniq, quads


@pytest.mark.parametrize("name", ["criteo_b256", "large_t4_b256"])
def test_bf16_gradients_sum_like_their_fp32_widening(name):
    say("bf16 grads", name)
    w, uniq, quads = _bags_and_unique(name)
    B, T, d = w.batch, w.num_tables, w.dim
    U = uniq.size
    rng = np.random.default_rng(5)
    # small integers: exact in bf16, and every partial sum exact in fp32
    g16 = dev(rng.integers(-8, 9, size=(B, T + 1, d)).astype(np.float32)).to(torch.bfloat16)
    g32 = g16.float()
    nu = dev(np.array([U], np.int32))
    src = dev(quads)
    off = dev(w.offsets)
    args = ((T + 1) * d, d, off, B, T, d, None, None, nu)
    r16 = ctr.ctr_embbag_bwd(g16[:, 1:, :], *args, sorted_src=src, nnz=w.nnz)
    r32 = ctr.ctr_embbag_bwd(g32[:, 1:, :], *args, sorted_src=src, nnz=w.nnz)
    np.testing.assert_array_equal(host(r16)[:U], host(r32)[:U])
    uq = dev(uniq)
    for sr in (False, True):
        ta = gpu_table(w.rows, d, w.dtype, 9)
        tb = gpu_table(w.rows, d, w.dtype, 9)
        if sr:
            ctr.ctr_embbag_bwd_sgd(g16[:, 1:, :], (T + 1) * d, d, off, B, T, w.nnz, src, nu,
                                   ta, uq, 0.05, rounding=ctr.CTR_ROUND_STOCHASTIC, seed=1234)
            ctr.ctr_embbag_bwd_sgd(g32[:, 1:, :], (T + 1) * d, d, off, B, T, w.nnz, src, nu,
                                   tb, uq, 0.05, rounding=ctr.CTR_ROUND_STOCHASTIC, seed=1234)
        else:
            ctr.ctr_embbag_bwd_sgd(g16[:, 1:, :], (T + 1) * d, d, off, B, T, w.nnz, src, nu,
                                   ta, uq, 0.05)
            ctr.ctr_embbag_bwd_sgd(g32[:, 1:, :], (T + 1) * d, d, off, B, T, w.nnz, src, nu,
                                   tb, uq, 0.05)
        assert torch.equal(ta, tb), sr
    # random values: the bf16 path against the oracle's sums of the widened values
    gr = dev(rng.standard_normal((B, T + 1, d)).astype(np.float32)).to(torch.bfloat16)
    rr = ctr.ctr_embbag_bwd(gr[:, 1:, :], *args, sorted_src=src, nnz=w.nnz)
    keys = orc.form_keys(w.indices, w.offsets, T, B, w.row_base)
    _, inv, _, _ = orc.unique(keys)
    want, mag = orc.embbag_bwd(host(gr)[:, 1:, :].astype(np.float64), w.offsets, B, T, inv, U)
    assert_close(host(rr)[:U], want, mag, gamma(segreduce_depth(w.nnz, d, True)),
                 "bf16 row sums")


def _synthetic_bags(T, B, rows, seed):
    """Bags of 0-12 rows over T tables, plus one hot row per table that many bags hold (its
    segment crosses slots, chunks and carry levels), with the (u, bag, row) quadruples of the
    sorted occurrences from the oracle's unique."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 13, size=(T, B))
    lens[rng.random((T, B)) < 0.1] = 0
    idx = []
    for t in range(T):
        for b in range(B):
            r = rng.integers(0, rows[t], size=int(lens[t, b]))
            if lens[t, b] and rng.random() < 0.6:
                r[0] = 3                              # the hot row of table t
            idx.append(r)
    off = np.zeros(T * B + 1, dtype=np.int64)
    off[1:] = np.cumsum(lens.reshape(-1))
    ids = np.concatenate(idx).astype(np.int64)
    row_base = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    keys = orc.form_keys(ids, off, T, B, row_base)
    uniq, inv, perm, _ = orc.unique(keys)
    n = ids.size
    bag_of = np.searchsorted(off, np.arange(n), side="right") - 1
    quads = np.zeros((n, 4), dtype=np.int32)
    quads[:, 0], quads[:, 1] = inv[perm], bag_of[perm]
    quads[:, 2:] = uniq[inv[perm]].astype(np.int64).view(np.int32).reshape(-1, 2)
    return ids, off, uniq, inv, quads


# bf16 gradient rows are read 8 columns per lane at the first level when dim is a multiple of
# 8 up to 512 (1 to 64 lanes per row); other widths take 4 columns per lane
@pytest.mark.parametrize("dtype,d", [("bf16", 8), ("bf16", 16), ("bf16", 24), ("bf16", 32),
                                     ("bf16", 40), ("bf16", 64), ("bf16", 96), ("bf16", 200),
                                     ("bf16", 256), ("bf16", 384), ("bf16", 512),
                                     ("bf16", 1024), ("f32", 4), ("f32", 12), ("f32", 8),
                                     ("f16", 48)])
def test_bf16_gradient_rows_every_width(dtype, d):
    T, B = 3, 97
    rows = [700, 300, 900]
    ids, off, uniq, inv, quads = _synthetic_bags(T, B, rows, d)
    n, U = ids.size, uniq.size
    say("bf16 grads width", dtype, d, n, U)
    rng = np.random.default_rng(d + 11)
    nu = dev(np.array([U], np.int32))
    src, offd = dev(quads), dev(off)
    args = (T * d, d, offd, B, T, d, None, None, nu)
    # small integers: exact in bf16 and in every fp32 partial sum, so the 8-column lanes
    # and the fp32 rows' 4-column lanes (other slot depths) give the same bits
    g16 = dev(rng.integers(-8, 9, size=(B, T, d)).astype(np.float32)).to(torch.bfloat16)
    g32 = g16.float()
    r16 = ctr.ctr_embbag_bwd(g16, *args, sorted_src=src, nnz=n)
    r32 = ctr.ctr_embbag_bwd(g32, *args, sorted_src=src, nnz=n)
    np.testing.assert_array_equal(host(r16)[:U], host(r32)[:U])
    uq = dev(uniq)
    for rounding in (ctr.CTR_ROUND_NEAREST, ctr.CTR_ROUND_STOCHASTIC):
        if rounding == ctr.CTR_ROUND_STOCHASTIC and dtype == "f32":
            continue
        ta, tb = gpu_table(rows, d, dtype, 9), gpu_table(rows, d, dtype, 9)
        before = ta.clone()
        for g, t in ((g16, ta), (g32, tb)):
            ctr.ctr_embbag_bwd_sgd(g, T * d, d, offd, B, T, n, src, nu, t, uq, 0.05,
                                   rounding=rounding, seed=4321)
        assert torch.equal(ta, tb), rounding
        assert not torch.equal(ta, before)
    # random values against the oracle's sums of the widened values
    gr = dev(rng.standard_normal((B, T, d)).astype(np.float32)).to(torch.bfloat16)
    rr = ctr.ctr_embbag_bwd(gr, *args, sorted_src=src, nnz=n)
    want, mag = orc.embbag_bwd(host(gr).astype(np.float64), off, B, T, inv, U)
    assert_close(host(rr)[:U], want, mag, gamma(segreduce_depth(n, d, True)),
                 "bf16 row sums, d=%d" % d)
