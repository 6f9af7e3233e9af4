"""binary16 table storage ("DHEN" notes, 6.4 "Common Optimizations": FP16 embeddings with
stochastic rounding) on the GPU, through the C ABI.

* The stores at their edges: a zero table updated with lr = 1 stores round(x) for chosen
  binary32 x (every tie class, the subnormal range, the overflow threshold, NaN and
  infinities), nearest-even and stochastic, bit for bit against the oracle's rounding of the
  same x with the same random bits.
* ctr_sparse_sgd with CTR_ROUND_STOCHASTIC on a binary16 table, bit for bit against the
  oracle, over gradients of six decades.
* The fused backward + SGD leaves a binary16 table bit-identical to the two-call path, both
  roundings; a training step end to end against the oracle's chain within the derived
  bounds; the native step runner matches the Python-driven step.
Pooling, the table fill and the row gathers of binary16 tables are in test_gpu_parity.py.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from sparse_embedding_lookup_amd import ctr, workloads
from sparse_embedding_lookup_amd.pipeline import SR_SEED, FrontEnd
from tests.chain import check_chain, oracle_dlrm_step
from tests.test_gpu_parity import DEV, dev, gpu_table, host, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DIM = 8


def _edge_values():
    """binary32 values at the edges of binary16 rounding, both signs."""
    grid = np.arange(1, 0x7C00, 97, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = (np.arange(1, 0x7C00, 97, dtype=np.uint16) + 1).view(np.float16).astype(np.float64)
    mids = (grid + nxt) / 2.0                                   # ties (exact in binary32)
    sub = np.arange(0, 1025, 7) * 2.0 ** -24                    # subnormal grid
    sub_mid = (np.arange(0, 1024, 7) + 0.5) * 2.0 ** -24        # subnormal ties
    rng = np.random.default_rng(5)
    rand = 2.0 ** rng.uniform(-30, 16.5, 3000)
    near_max = [65504.0, 65505.0, 65519.0, 65519.99, 65520.0, 65521.0, 65535.0, 65536.0, 1e5,
                3e38, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -30, 2.0 ** -25, 2.0 ** -25 * 1.0001,
                1e-40, 1e-45]
    v = np.concatenate([grid, mids, sub, sub_mid, rand, near_max])
    # no -0: x = fmaf(-1, -v, +0) is +0 for v = -0, so -0 cannot be stored this way
    v = np.concatenate([v, -v[v != 0]]).astype(np.float32)
    pad = (-v.size) % DIM
    return np.concatenate([v, np.full(pad, 0.5, np.float32)]).reshape(-1, DIM)


def _store_through_sgd(vals, rounding, seed):
    """A zero binary16 table, row u updated with lr = 1 and g = -vals[u]: the kernel stores
    its rounding of fmaf(-1, g, 0) = vals[u] exactly."""
    n = vals.shape[0]
    t = torch.zeros((n, DIM), dtype=torch.float16, device=DEV)
    uq = np.arange(n, dtype=np.int64)
    g = (-vals).astype(np.float32)
    ctr.ctr_sparse_sgd(t, dev(uq), dev(np.array([n], np.int32)), n, dev(g), 1.0, rounding, seed)
    return host(t).astype(np.float64)


def _same(got, want):
    both_nan = np.isnan(got) & np.isnan(want)
    ok = (got == want) | both_nan
    # the sign of a zero is part of the stored value
    ok &= (np.signbit(got) == np.signbit(want)) | both_nan
    assert ok.all(), (np.argwhere(~ok)[:5], got[~ok][:5], want[~ok][:5])


def test_f16_nearest_store_edges():
    vals = _edge_values()
    say("f16 nearest edges", vals.size)
    got = _store_through_sgd(vals, ctr.CTR_ROUND_NEAREST, 0)
    want = np.vectorize(orc.round_f16)(vals.astype(np.float64))
    _same(got, want)
    # NaN and infinity inputs
    special = np.array([[np.nan, np.inf, -np.inf, 0.0, 1.0, -1.0, 7.0, 65504.0]], np.float32)
    got = _store_through_sgd(special, ctr.CTR_ROUND_NEAREST, 0)
    _same(got, np.vectorize(orc.round_f16)(special.astype(np.float64)))


@pytest.mark.parametrize("seed", [1, 0xDEADBEEF12345678])
def test_f16_stochastic_store_edges(seed):
    vals = _edge_values()
    say("f16 stochastic edges", seed)
    got = _store_through_sgd(vals, ctr.CTR_ROUND_STOCHASTIC, seed)
    n = vals.shape[0]
    want = np.empty_like(got)
    for u in range(n):
        for c in range(DIM):
            want[u, c] = orc.sr_f16(float(vals[u, c]), orc.sr_bits(seed, u, c, DIM))
    _same(got, want)
    # both neighbours occur where a value sits between two binary16 values
    inexact = np.vectorize(orc.round_f16)(vals.astype(np.float64)) != vals
    assert 0.2 < np.mean((got > vals)[inexact & np.isfinite(got)]) < 0.8


@pytest.mark.parametrize("dim", [8, 64, 1024])
def test_sparse_sgd_sr_f16_bit_exact(dim):
    say("sgd sr f16", dim)
    rows = [4000, 3001]
    t = gpu_table(rows, dim, "f16", 31)
    before = host(t)
    tab = orc.Table(rows, dim, "f16", 31)
    rng = np.random.default_rng(dim + 1)
    U = 1501
    uniq = np.sort(rng.choice(7001, size=U, replace=False)).astype(np.int64)
    g = (rng.standard_normal((U, dim)) * 10.0 ** rng.integers(-4, 2, size=(U, 1))).astype(
        np.float32)
    cap = U + 64
    uq = np.zeros(cap, np.int64)
    uq[:U] = uniq
    gg = np.zeros((cap, dim), np.float32)
    gg[:U] = g
    seed = 0xF16 ^ dim
    ctr.ctr_sparse_sgd(t, dev(uq), dev(np.array([U], np.int32)), cap, dev(gg), 0.01,
                       ctr.CTR_ROUND_STOCHASTIC, seed)
    after = host(t)
    np.testing.assert_array_equal(after[uniq], orc.sparse_sgd_sr(tab, uniq, g, 0.01, seed))
    untouched = np.ones(sum(rows), bool)
    untouched[uniq] = False
    np.testing.assert_array_equal(after[untouched], before[untouched])


def _f16_workload(name):
    w = {"small_b256": lambda: workloads.small(batch=256),
         "criteo_b128": lambda: workloads.criteo(batch=128)}[name]()
    return dataclasses.replace(w, dtype="f16")


@pytest.mark.parametrize("rounding", ["nearest", "stochastic"])
@pytest.mark.parametrize("name", ["small_b256", "criteo_b128"])
def test_fused_bwd_sgd_f16_matches_two_calls(name, rounding):
    w = _f16_workload(name)
    say("fused bwd+sgd f16", name, rounding)
    fa = FrontEnd(w, DEV, fused=True, keep_grads=True, rounding=rounding)
    fb = FrontEnd(w, DEV, fused=False, rounding=rounding)
    assert fa.table.dtype == torch.float16
    before = fa.table.clone()
    fa.step()
    fb.step()
    U = int(host(fa.num_unique)[0])
    np.testing.assert_array_equal(host(fa.row_grads)[:U], host(fb.row_grads)[:U])
    assert torch.equal(fa.table, fb.table)
    assert not torch.equal(fa.table, before)
    if rounding == "stochastic":
        # from the kernel's own binary32 row gradients, the oracle's update is the kernel's
        tab = orc.Table(w.rows, w.dim, w.dtype, w.table_seed)
        uniq = host(fa.uniq)[:U]
        seed0 = orc.splitmix64_stream(SR_SEED, 1)[0]
        want = orc.sparse_sgd_sr(tab, uniq, host(fa.row_grads)[:U], w.lr, seed0)
        np.testing.assert_array_equal(host(fa.table[fa.uniq[:U]]), want)


@pytest.mark.parametrize("name", ["small_b256", "criteo_b128"])
def test_end_to_end_f16_step(name):
    w = _f16_workload(name)
    say("end_to_end f16", name, w.nnz)
    fe = FrontEnd(w, DEV, keep_grads=True)
    fe.step()
    check_chain(w, fe, oracle_dlrm_step(w))


@pytest.mark.parametrize("schedule", ["serial", "overlap"])
def test_native_step_f16_matches_python_steps(schedule):
    w = _f16_workload("small_b256")
    say("native step f16", schedule)
    pipelined = schedule != "serial"
    fa = FrontEnd(w, DEV, keep_grads=True, pipelined=pipelined, rounding="stochastic")
    fb = FrontEnd(w, DEV, keep_grads=True, pipelined=pipelined, rounding="stochastic")
    if pipelined:
        fa.pipeline_start()
        fb.native_start()
    for k in range(2):
        if pipelined:
            fa.step_pipelined(fork_after="embbag_fwd")
        else:
            fa.step()
        fb.step_native(schedule)
        torch.cuda.synchronize()
        U = int(host(fa.num_unique)[0])
        np.testing.assert_array_equal(host(fa.row_grads)[:U], host(fb.row_grads)[:U])
        assert torch.equal(fa.table, fb.table), k
