"""The bf16 gradient of a bf16 interaction: the MFMA backward stores dZ rounded to bf16, and
the pooling's backward reads bf16 gradient rows and sums them in fp32.

* The bf16 dZ is exactly the fp32 dZ of the same kernel rounded to nearest-even: same
  arithmetic, only the store differs.
* Row sums from bf16 gradients equal the row sums of the same values widened to fp32, bit
  for bit, when the values are small integers.  Their fp32 sums are exact in any order, and
  the two dtypes use different slot depths.  This holds for row gradients only, with the
  nearest-even update, and with stochastic rounding.  For random values the bf16 path
  matches the oracle within rtol * M.
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
