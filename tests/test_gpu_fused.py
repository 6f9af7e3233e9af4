"""Parity of the fused forward (ctr_embbag_interaction_fwd: pooling into Z and the dot
interaction from an on-chip copy) with the oracle, through the C ABI.

Every case is checked three ways:
  * Z's pooled rows against the oracle's pooling of the same table and bags (rtol fp32);
  * R against the oracle's interaction of the kernel's own Z, the input its second phase
    reads (rtol of the compute type), and R[:, :dim] equal to the dense rows bit for bit;
  * R against the oracle's whole chain (pooling, then interaction): 3 rtol, the bar of the
    separate calls' end-to-end tests.
Cases span one- and multi-sample blocks with a ragged last block, empty bags, a bag longer
than a block's lane-group shares, F from 2 to 65 (one to three 32-row tiles, a ragged last
tile), mixed table and compute types, int32 and int64 indices, and the full-size workloads.
"""
import zlib

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from sparse_embedding_lookup_amd import ctr, workloads
from sparse_embedding_lookup_amd.pipeline import FrontEnd
from tests.chain import check_chain, oracle_dlrm_step
from tests.parity import assert_close, assert_within, gamma, pool_eps, step_bounds
from tests.test_gpu_parity import DEV, dev, gpu_table, host, rand_csr, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _case(name):
    """rows, dim, table dtype, compute, ids, offsets, batch, tables."""
    rng = np.random.default_rng(zlib.crc32(name.encode()))

    def from_w(w, compute=None):
        return (w.rows, w.dim, w.dtype, compute or w.compute, w.indices, w.offsets, w.batch,
                w.num_tables)

    if name == "tiny":
        return from_w(workloads.tiny())
    if name == "small_b256":
        return from_w(workloads.small(batch=256))
    if name == "criteo_b128":
        return from_w(workloads.criteo(batch=128))
    if name == "large_b48":
        return from_w(workloads.large(batch=48, rows=5000))
    if name == "small_b6145":          # three samples per block, one in the last
        return from_w(workloads.small(batch=6145, rows=100_000))
    if name == "criteo_b6145":
        return from_w(workloads.criteo(batch=6145, row_scale=0.01))
    if name == "small_bf16_compute":   # fp32 table, matrix-core dots
        return from_w(workloads.small(batch=300), "bf16")
    if name == "criteo_f32_compute":   # bf16 table, fp32 dots
        return from_w(workloads.criteo(batch=200), "f32")
    if name == "empty_bags_d64":
        rows = [100, 3000, 7]
        ids, off = rand_csr(rng, 3, 333, rows, 9, empty_frac=0.3)
        return rows, 64, "f32", "f32", ids, off, 333, 3
    if name == "all_empty":
        off = np.zeros(4 * 50 + 1, dtype=np.int64)
        return [10, 10, 10, 10], 32, "bf16", "bf16", np.zeros(0, np.int64), off, 50, 4
    if name == "long_bags_d128":       # bags of up to 3000 rows cross many group shares
        rows = [20_000, 500]
        ids, off = rand_csr(rng, 2, 5, rows, 3000)
        return rows, 128, "bf16", "bf16", ids, off, 5, 2
    if name == "f2_d32":               # F = 2: one pair
        rows = [1000]
        ids, off = rand_csr(rng, 1, 77, rows, 5)
        return rows, 32, "bf16", "bf16", ids, off, 77, 1
    if name == "f33_d16":              # second tile row holds one vector: no pair inside it
        rows = [50] * 32
        ids, off = rand_csr(rng, 32, 41, rows, 3)
        return rows, 16, "bf16", "bf16", ids, off, 41, 32
    if name == "f65_f32_d128":         # the largest fp32 copy that fits one block
        rows = [200] * 64
        ids, off = rand_csr(rng, 64, 9, rows, 4)
        return rows, 128, "bf16", "f32", ids, off, 9, 64
    if name == "f9_f32_d4":            # one lane per row
        rows = [30] * 8
        ids, off = rand_csr(rng, 8, 500, rows, 6, empty_frac=0.1)
        return rows, 4, "f32", "f32", ids, off, 500, 8
    raise KeyError(name)


CASES = ["tiny", "small_b256", "criteo_b128", "large_b48", "small_b6145", "criteo_b6145",
         "small_bf16_compute", "criteo_f32_compute", "empty_bags_d64", "all_empty",
         "long_bags_d128", "f2_d32", "f33_d16", "f65_f32_d128", "f9_f32_d4"]


def _run_fused(rows, dim, dtype, compute, ids, off, B, T, itype="i64", seed=7):
    t = gpu_table(rows, dim, dtype, seed)
    tab = orc.Table(rows, dim, dtype, seed)
    rng = np.random.default_rng(seed)
    dense = rng.standard_normal((B, dim)).astype(np.float32)
    F = T + 1
    Z = torch.full((B, F, dim), float("nan"), dtype=torch.float32, device=DEV)
    Z[:, 0, :] = dev(dense)
    code = ctr.CTR_BF16 if compute == "bf16" else ctr.CTR_F32
    gi = dev(ids.astype(np.int32 if itype == "i32" else np.int64))
    R = torch.full((B, dim + F * (F - 1) // 2), float("nan"), dtype=torch.float32, device=DEV)
    ctr.ctr_embbag_interaction_fwd(t, gi, dev(off), Z, code, R, row_base=dev(tab.row_base))
    return tab, dense, host(Z), host(R)


def _check(name, tab, dense, ids, off, B, compute, Zg, Rg):
    T = tab.num_tables
    d = dense.shape[1]
    pooled, pmag = orc.embbag_fwd(tab, ids, off, B)
    assert_within(Zg[:, 1:], pooled, pool_eps(off, B, T) * pmag, "fused Z " + name, mag=pmag)
    np.testing.assert_array_equal(Zg[:, 0], dense)
    np.testing.assert_array_equal(Rg[:, :d], dense)
    # the interaction step on its own input: for matrix-core dots the oracle rounds the same
    # operands to bf16, so only the fp32 accumulation over d columns differs
    want, mag = orc.interaction_fwd(Zg.astype(np.float64), bf16=compute == "bf16")
    assert_close(Rg, want, mag, gamma(d), "fused R (own Z) " + name)
    # the whole chain
    Z = np.concatenate([dense[:, None, :].astype(np.float64), pooled], axis=1)
    Zm = np.concatenate([np.abs(dense[:, None, :]).astype(np.float64), pmag], axis=1)
    want, mag = orc.interaction_fwd(Z, Zm)
    lmax = int(np.diff(off).max()) if len(ids) else 0
    eR = step_bounds(lmax, d, T + 1, len(ids), compute == "bf16", False)["R"]
    assert_close(Rg, want, mag, eR, "fused R (chain) " + name)


@pytest.mark.parametrize("name", CASES)
def test_fused_forward_matches_oracle(name):
    rows, dim, dtype, compute, ids, off, B, T = _case(name)
    say("embbag_interaction_fwd", name, B, T, dim, dtype, compute, len(ids))
    tab, dense, Zg, Rg = _run_fused(rows, dim, dtype, compute, ids, off, B, T)
    _check(name, tab, dense, ids, off, B, compute, Zg, Rg)


@pytest.mark.parametrize("name", ["criteo_b128", "empty_bags_d64", "f9_f32_d4"])
def test_fused_forward_int32_indices(name):
    rows, dim, dtype, compute, ids, off, B, T = _case(name)
    say("embbag_interaction_fwd i32", name)
    tab, dense, Zg, Rg = _run_fused(rows, dim, dtype, compute, ids, off, B, T, itype="i32")
    _check(name, tab, dense, ids, off, B, compute, Zg, Rg)


def test_fused_forward_empty_batch():
    t = gpu_table([10], 16, "f32", 1)
    Z = torch.zeros((0, 2, 16), device=DEV)
    R = torch.zeros((0, 17), device=DEV)
    ctr.ctr_embbag_interaction_fwd(t, dev(np.zeros(0, np.int64)), dev(np.zeros(1, np.int64)), Z,
                                   ctr.CTR_F32, R)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["tiny", "small_b256", "criteo_b128"])
def test_fused_step_end_to_end(name):
    """A whole training step whose forward is the fused call, against the oracle's chain
    (the bounds of the separate calls' end-to-end test)."""
    w = {"tiny": workloads.tiny, "small_b256": lambda: workloads.small(batch=256),
         "criteo_b128": lambda: workloads.criteo(batch=128)}[name]()
    say("fused step end to end", name)
    fe = FrontEnd(w, DEV, keep_grads=True, fused_fwd=True)
    assert [n for n, _ in fe.stages()][0] == "embbag_interaction_fwd"
    fe.step()
    check_chain(w, fe, oracle_dlrm_step(w))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["small", "criteo"])
def test_fused_forward_full_size(name):
    """The bench's workloads at full size, every output checked."""
    w = workloads.make(name)
    say("fused full size", name, w.nnz)
    fe = FrontEnd(w, DEV, fused_fwd=True)
    fe.forward()
    Zg, Rg = host(fe.Z), host(fe.R)
    say("oracle", name)
    tab = orc.Table(w.rows, w.dim, w.dtype, w.table_seed)
    _check(name, tab, w.dense, w.indices, w.offsets, w.batch, w.compute, Zg, Rg)
