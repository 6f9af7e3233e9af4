"""Stochastic rounding of the bf16 sparse update ("DHEN" notes, 6.4 "Common Optimizations")
on the GPU, through the C ABI.

* ctr_sparse_sgd with CTR_ROUND_STOCHASTIC against the oracle, bit for bit.  Both sides take the rounding decision
  on the same binary32 value, a fused multiply-add, with the same counter-based bits.
* The fused backward, ctr_embbag_bwd_sgd with CTR_ROUND_STOCHASTIC, is bit-identical to
  ctr_embbag_bwd followed by ctr_sparse_sgd with the same rounding and seed.  Every value it stores is a bf16 neighbour of the
  oracle's exact update.
* ctr_step_run with rounding = CTR_ROUND_STOCHASTIC matches the same steps driven call by
  call, with the same per-step seeds.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from sparse_embedding_lookup_amd import ctr, workloads
from sparse_embedding_lookup_amd.pipeline import SR_SEED, FrontEnd
from tests.parity import step_bounds
from tests.test_gpu_parity import DEV, dev, gpu_table, host, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("dim", [8, 64, 128, 512, 1024, 2048])
def test_sparse_sgd_sr_bit_exact(dim):
    say("sgd sr", dim)
    rows = [4000, 3001]
    t = gpu_table(rows, dim, "bf16", 31)
    before = host(t.float())
    tab = orc.Table(rows, dim, "bf16", 31)
    rng = np.random.default_rng(dim)
    U = 1501
    uniq = np.sort(rng.choice(7001, size=U, replace=False)).astype(np.int64)
    # gradients over six decades, so that many updates are far below half an ulp
    g = (rng.standard_normal((U, dim)) * 10.0 ** rng.integers(-4, 2, size=(U, 1))).astype(
        np.float32)
    cap = U + 64
    uq = np.zeros(cap, np.int64)
    uq[:U] = uniq
    gg = np.zeros((cap, dim), np.float32)
    gg[:U] = g
    seed = 0xC0FFEE ^ dim
    ctr.ctr_sparse_sgd(t, dev(uq), dev(np.array([U], np.int32)), cap, dev(gg), 0.01,
                       ctr.CTR_ROUND_STOCHASTIC, seed)
    after = host(t.float())
    want = orc.sparse_sgd_sr(tab, uniq, g, 0.01, seed)
    np.testing.assert_array_equal(after[uniq], want)
    untouched = np.ones(sum(rows), bool)
    untouched[uniq] = False
    np.testing.assert_array_equal(after[untouched], before[untouched])
    # the stochastic choice is live: nearest-even from the same start differs somewhere
    near = orc.sparse_sgd(tab, uniq, g.astype(np.float64), np.abs(g).astype(np.float64), 0.01)[0]
    assert np.any(want != near)


def _bf16_workload(name):
    if name == "criteo_b128":
        return workloads.criteo(batch=128)
    if name == "criteo_b1024":
        return workloads.criteo(batch=1024)
    if name == "large_t4_b256":
        return workloads.large(batch=256, tables=4, rows=20_000)
    raise KeyError(name)


def _ulp_bf16(x):
    """Spacing of bfloat16 values at |x| (8 significant bits), at least the subnormal one."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("name", ["criteo_b128", "criteo_b1024", "large_t4_b256"])
def test_fused_bwd_sgd_sr_matches_two_calls_and_oracle(name):
    w = _bf16_workload(name)
    say("fused bwd+sgd sr", name)
    fa = FrontEnd(w, DEV, fused=True, keep_grads=True, rounding="stochastic")
    fb = FrontEnd(w, DEV, fused=False, rounding="stochastic")
    fa.step()
    fb.step()
    U = int(host(fa.num_unique)[0])
    np.testing.assert_array_equal(host(fa.row_grads)[:U], host(fb.row_grads)[:U])
    assert torch.equal(fa.table, fb.table)
    # every updated value is a bf16 neighbour of the oracle's exact w - lr * g
    tab = orc.Table(w.rows, w.dim, w.dtype, w.table_seed)
    pooled, pmag = orc.embbag_fwd(tab, w.indices, w.offsets, w.batch)
    B, F, d = w.batch, w.F, w.dim
    Z = np.empty((B, F, d))
    Zm = np.empty((B, F, d))
    Z[:, 0], Zm[:, 0] = w.dense, np.abs(w.dense)
    Z[:, 1:], Zm[:, 1:] = pooled, pmag
    dZ, dZm = orc.interaction_bwd(Z, w.grad_out.astype(np.float64), Zm)
    keys = orc.form_keys(w.indices, w.offsets, w.num_tables, B, w.row_base)
    uniq, inv, _, _ = orc.unique(keys)
    g, gm = orc.embbag_bwd(dZ[:, 1:], w.offsets, B, w.num_tables, inv, uniq.size, dZm[:, 1:])
    stored = orc.gather_rows(tab, uniq)
    x = stored - w.lr * g
    got = host(fa.table[fa.uniq[:U]].float()).astype(np.float64)
    np.testing.assert_array_equal(host(fa.uniq)[:U], uniq)
    # the gradient carries the chain's error (bf16 operands, a bf16-stored dZ, the tree)
    eg = step_bounds(int(np.diff(w.offsets).max()), d, F, w.nnz, w.compute == "bf16",
                     fa.dZ.dtype == torch.bfloat16)["g"]
    bound = 2 * _ulp_bf16(x) + w.lr * eg * gm
    err = np.abs(got - x)
    assert np.all(err <= bound), (err / bound).max()
    # and a genuine mix of both neighbours, not one systematic direction
    assert 0.2 < np.mean(got > x) < 0.8
    # from the kernel's own binary32 row gradients, the oracle's update (seed of step 0 from
    # the oracle's generator) is the fused kernel's, bit for bit
    seed0 = orc.splitmix64_stream(SR_SEED, 1)[0]
    want = orc.sparse_sgd_sr(tab, uniq, host(fa.row_grads)[:U], w.lr, seed0)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("schedule", ["serial", "overlap"])
def test_native_step_sr_matches_python_steps(schedule):
    w = workloads.criteo(batch=128)
    say("native step sr", schedule)
    pipelined = schedule != "serial"
    fa = FrontEnd(w, DEV, keep_grads=True, pipelined=pipelined, rounding="stochastic")
    fb = FrontEnd(w, DEV, keep_grads=True, pipelined=pipelined, rounding="stochastic")
    fc = FrontEnd(w, DEV, keep_grads=True)                  # nearest-even, for contrast
    if pipelined:
        fa.pipeline_start()
        fb.native_start()
    for k in range(3):
        if pipelined:
            fa.step_pipelined(fork_after="embbag_fwd")
        else:
            fa.step()
        fb.step_native(schedule)
        fc.step()
        torch.cuda.synchronize()
        U = int(host(fa.num_unique)[0])
        np.testing.assert_array_equal(host(fa.row_grads)[:U], host(fb.row_grads)[:U])
        assert torch.equal(fa.table, fb.table), k
        assert not torch.equal(fa.table, fc.table)
