"""Parity at the workloads' full sizes, in the configuration bench.py times (fused backward +
SGD, unique on the side stream).

Tiny, Small, Criteo and TensorNet run the whole step on both sides.  Large (65.5 GB of bf16
tables, 67M occurrences) is checked on sampled outputs the oracle computes one by one
(pooled bags, interaction rows of sampled samples, per-row gradients and updated rows of
sampled keys) and on properties that hold at any size (unique/inverse/perm invariants against
numpy.unique).
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from sparse_embedding_lookup_amd import ctr, workloads
from sparse_embedding_lookup_amd.pipeline import FrontEnd
from tests.chain import check_chain, oracle_dlrm_step
from tests.parity import (assert_close, assert_within, gamma, segreduce_depth, sgd_store_bound,
                          step_bounds, store_bound)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:               # numpy has no bfloat16: widen (exact)
        t = t.float()
    return t.detach().cpu().numpy()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def check_unique_properties(keys, fe):
    """GPU unique outputs against numpy.unique and the invariants, at any size."""
    n = keys.size
    U = int(host(fe.num_unique)[0])
    uniq = host(fe.uniq[:max(U, 1)])[:U]
    inv = host(fe.inverse[:n])
    perm = host(fe.perm[:n])
    seg = host(fe.seg[:U + 1])
    u2, cnt = np.unique(keys, return_counts=True)
    assert U == u2.size
    np.testing.assert_array_equal(uniq, u2)
    np.testing.assert_array_equal(np.diff(seg), cnt)
    np.testing.assert_array_equal(uniq[inv], keys)
    sk = keys[perm]
    d = np.diff(sk)
    assert np.all(d >= 0)
    assert np.all(np.diff(perm.astype(np.int64))[d == 0] > 0)      # stable
    assert np.array_equal(np.bincount(perm, minlength=n), np.ones(n, np.int64))
    return uniq, inv


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny", "small", "criteo"])
def test_full_dlrm_step(name):
    w = workloads.make(name)
    say("full step", name, "nnz", w.nnz)
    fe = FrontEnd(w, DEV, keep_grads=True)
    fe.step()
    torch.cuda.synchronize()
    say("oracle", name)
    o = oracle_dlrm_step(w)
    check_chain(w, fe, o)
    uniq, inv = check_unique_properties(o["keys"], fe)
    # rows outside the batch are untouched: compare a sample against the fill definition
    rng = np.random.default_rng(5)
    cand = rng.integers(0, w.total_rows, 4000)
    cand = cand[~np.isin(cand, o["uniq"])][:2000]
    tab = orc.Table(w.rows, w.dim, w.dtype, w.table_seed)
    np.testing.assert_array_equal(host(fe.table[dev(cand)].float()), orc.table_rows(tab, cand))


@pytest.mark.timeout(600)
def test_full_tensornet_step():
    w = workloads.tensornet()
    say("full step tensornet nnz", w.nnz)
    fe = FrontEnd(w, DEV, keep_grads=True)
    fe.step()
    torch.cuda.synchronize()
    tab = orc.Table(w.rows, w.dim, w.dtype, w.table_seed)
    keys = orc.form_keys(w.indices, w.offsets, 1, w.nnz, np.array([0, w.rows[0]]), w.key_modulus)
    say("oracle unique")
    uniq, inv, perm, seg = orc.unique(keys)
    U = uniq.size
    u_gpu, i_gpu = check_unique_properties(keys, fe)
    np.testing.assert_array_equal(u_gpu, uniq)
    np.testing.assert_array_equal(i_gpu, inv)
    np.testing.assert_array_equal(host(fe.perm[:w.nnz]), perm)
    E = orc.gather_rows(tab, uniq)
    np.testing.assert_array_equal(host(fe.E[:U]), E)
    out = host(fe.out[:w.nnz])
    np.testing.assert_array_equal(out, E[inv])          # per-slot vectors: exact row copies
    dout = w.grad_out.reshape(w.nnz, 1, w.dim).astype(np.float64)
    g, gm = orc.embbag_bwd(dout, w.offsets, w.nnz, 1, inv, U)
    eg = gamma(segreduce_depth(w.nnz, w.dim, False))
    assert_close(host(fe.row_grads[:U]), g, gm, eg, "tensornet row grads")
    new, nm = orc.sparse_sgd(tab, uniq, g, gm, w.lr)
    assert_within(host(fe.table[dev(uniq)]), new, sgd_store_bound(new, gm, w.lr, eg, False),
                  "tensornet rows", mag=nm)


@pytest.fixture(scope="module")
def large_run():
    say("generating Large")
    w = workloads.large()
    say("Large nnz", w.nnz)
    fe = FrontEnd(w, DEV, keep_grads=True)
    # the fused forward at full size, into buffers of its own, before the step's update
    fe.fused_Z = fe.Z.clone()                  # row 0 of each sample: the dense vector
    fe.fused_R = torch.empty_like(fe.R)
    ctr.ctr_embbag_interaction_fwd(fe.table, fe.indices, fe.offsets, fe.fused_Z, fe.compute,
                                   fe.fused_R, row_base=fe.row_base)
    torch.cuda.synchronize()
    say("Large fused forward done")
    fe.step()
    torch.cuda.synchronize()
    say("Large step done")
    yield w, fe
    del fe
    torch.cuda.empty_cache()


def _sample_bags(w, k, seed):
    rng = np.random.default_rng(seed)
    return rng.choice(w.num_tables * w.batch, size=k, replace=False)


@pytest.mark.timeout(900)
def test_large_pooling_sampled(large_run):
    w, fe = large_run
    one = orc.Table(w.rows, w.dim, w.dtype, w.table_seed)   # rows regenerated by definition
    Z = host(fe.Z)
    for s in _sample_bags(w, 3000, 1):
        t, b = divmod(int(s), w.batch)
        lo, hi = int(w.offsets[s]), int(w.offsets[s + 1])
        # the bag alone: a CSR with one bag per table, only table t's non-empty
        off = np.zeros(w.num_tables + 1, dtype=np.int64)
        off[t + 1:] = hi - lo
        out, mag = orc.embbag_fwd(one, w.indices[lo:hi], off, 1)
        assert_close(Z[b, 1 + t], out[0, t], mag[0, t], gamma(hi - lo - 1),
                     "Large pooled bag %d" % s)


@pytest.mark.timeout(900)
def test_large_interaction_sampled(large_run):
    """Interaction rows of sampled samples: the oracle pools every table of those samples
    itself, then runs the interaction forward and backward for them."""
    w, fe = large_run
    rng = np.random.default_rng(2)
    samples = rng.choice(w.batch, size=24, replace=False)
    one = orc.Table(w.rows, w.dim, w.dtype, w.table_seed)
    R = host(fe.R)
    dZ = host(fe.dZ)
    grad_bf16 = fe.dZ.dtype == torch.bfloat16
    for b in samples:
        ids, lens = [], []
        for t in range(w.num_tables):
            s = t * w.batch + int(b)
            ids.append(w.indices[w.offsets[s]:w.offsets[s + 1]])
            lens.append(int(w.offsets[s + 1] - w.offsets[s]))
        off = np.zeros(w.num_tables + 1, dtype=np.int64)
        off[1:] = np.cumsum(lens)
        pooled, pmag = orc.embbag_fwd(one, np.concatenate(ids), off, 1)
        Z = np.concatenate([w.dense[b][None, None, :].astype(np.float64), pooled], axis=1)
        Zm = np.concatenate([np.abs(w.dense[b])[None, None, :].astype(np.float64), pmag], axis=1)
        eb = step_bounds(max(lens), w.dim, w.F, w.nnz, True, grad_bf16)
        Rw, Rm = orc.interaction_fwd(Z, Zm)
        assert_close(R[b][None], Rw, Rm, eb["R"], "Large R sample %d" % b)
        dZw, dZm = orc.interaction_bwd(Z, w.grad_out[b][None].astype(np.float64), Zm)
        assert_within(dZ[b][None], dZw, store_bound(dZw, dZm, eb["dZ"], grad_bf16),
                      "Large dZ sample %d" % b, mag=dZm)


@pytest.mark.timeout(900)
def test_large_fused_forward_sampled(large_run):
    """The fused pooling + interaction call at Large's full size: sampled samples' pooled
    rows and R rows against the oracle, which pools every table of those samples itself."""
    w, fe = large_run
    rng = np.random.default_rng(3)
    samples = rng.choice(w.batch, size=24, replace=False)
    one = orc.Table(w.rows, w.dim, w.dtype, w.table_seed)
    Zf = host(fe.fused_Z)
    Rf = host(fe.fused_R)
    for b in samples:
        ids, lens = [], []
        for t in range(w.num_tables):
            s = t * w.batch + int(b)
            ids.append(w.indices[w.offsets[s]:w.offsets[s + 1]])
            lens.append(int(w.offsets[s + 1] - w.offsets[s]))
        off = np.zeros(w.num_tables + 1, dtype=np.int64)
        off[1:] = np.cumsum(lens)
        pooled, pmag = orc.embbag_fwd(one, np.concatenate(ids), off, 1)
        pe = np.array([gamma(n - 1) for n in lens])[None, :, None]
        assert_within(Zf[b, 1:][None], pooled, pe * pmag, "Large fused Z sample %d" % b,
                      mag=pmag)
        np.testing.assert_array_equal(Rf[b, :w.dim], w.dense[b])
        Z = np.concatenate([w.dense[b][None, None, :].astype(np.float64), pooled], axis=1)
        Zm = np.concatenate([np.abs(w.dense[b])[None, None, :].astype(np.float64), pmag], axis=1)
        Rw, Rm = orc.interaction_fwd(Z, Zm)
        eR = step_bounds(max(lens), w.dim, w.F, w.nnz, True, False)["R"]
        assert_close(Rf[b][None], Rw, Rm, eR, "Large fused R sample %d" % b)


@pytest.mark.timeout(900)
def test_large_unique_properties(large_run):
    w, fe = large_run
    keys = orc.form_keys(w.indices, w.offsets, w.num_tables, w.batch, w.row_base)
    check_unique_properties(keys, fe)


@pytest.mark.timeout(900)
def test_large_backward_sampled(large_run):
    """Per-call parity of the backward at full size with GPU-independent inputs: the
    generator's N(0,1) gradient for every bag, reduced with the step's own grouping, checked
    on sampled rows (hot and cold) that the oracle sums over their occurrences."""
    w, fe = large_run
    rng = np.random.default_rng(3)
    B, T, d = w.batch, w.num_tables, w.dim
    dY = rng.standard_normal((B, T, d)).astype(np.float32)
    keys = orc.form_keys(w.indices, w.offsets, T, B, w.row_base)
    g_gpu = ctr.ctr_embbag_bwd(dev(dY), T * d, d, fe.offsets, B, T, d, None, None,
                               fe.num_unique, row_grads=fe.row_grads, sorted_src=fe.sorted_src,
                               nnz=w.nnz, workspace=fe.ws_bwd)
    U = int(host(fe.num_unique)[0])
    uniq = host(fe.uniq[:U])
    # sample distinct rows: the hottest ones and random ones
    counts = np.bincount(np.searchsorted(uniq, keys), minlength=U)
    pick = np.concatenate([np.argsort(-counts)[:20], rng.choice(U, 300, replace=False)])
    pick = np.unique(pick)
    occ = np.flatnonzero(np.isin(keys, uniq[pick]))
    bag = np.searchsorted(w.offsets, occ, side="right") - 1
    sub_inv = np.searchsorted(uniq[pick], keys[occ]).astype(np.int32)
    # the selected occurrences as one-occurrence bags over a [len(occ), 1, d] gradient
    sel = dY[bag % B, bag // B].astype(np.float64)[:, None, :]
    g, gm = orc.embbag_bwd(sel, np.arange(occ.size + 1, dtype=np.int64), occ.size, 1, sub_inv,
                           pick.size)
    got = host(g_gpu[dev(pick.astype(np.int64))])
    assert_close(got, g, gm, gamma(segreduce_depth(w.nnz, d, False)), "Large row grads")


@pytest.mark.timeout(900)
def test_large_sgd_sampled(large_run):
    """Updated rows of sampled keys: the oracle recomputes those rows' gradients over their
    occurrences from its own interaction backward of the samples involved."""
    w, fe = large_run
    rng = np.random.default_rng(4)
    U = int(host(fe.num_unique)[0])
    uniq = host(fe.uniq[:U])
    keys = orc.form_keys(w.indices, w.offsets, w.num_tables, w.batch, w.row_base)
    counts = np.bincount(np.searchsorted(uniq, keys), minlength=U)
    cold = np.flatnonzero(counts <= 2)
    pick = np.unique(rng.choice(cold, 40, replace=False))   # rows with few occurrences
    occ = np.flatnonzero(np.isin(keys, uniq[pick]))
    bag = np.searchsorted(w.offsets, occ, side="right") - 1
    one = orc.Table(w.rows, w.dim, w.dtype, w.table_seed)
    g = np.zeros((pick.size, w.dim))
    gm = np.zeros((pick.size, w.dim))
    cache = {}
    for o, s in zip(occ, bag):
        t, b = divmod(int(s), w.batch)
        if b not in cache:
            ids, lens = [], []
            for tt in range(w.num_tables):
                ss = tt * w.batch + b
                ids.append(w.indices[w.offsets[ss]:w.offsets[ss + 1]])
                lens.append(int(w.offsets[ss + 1] - w.offsets[ss]))
            off = np.zeros(w.num_tables + 1, dtype=np.int64)
            off[1:] = np.cumsum(lens)
            pooled, pmag = orc.embbag_fwd(one, np.concatenate(ids), off, 1)
            Z = np.concatenate([w.dense[b][None, None, :].astype(np.float64), pooled], axis=1)
            Zm = np.concatenate([np.abs(w.dense[b])[None, None, :].astype(np.float64), pmag], axis=1)
            cache[b] = orc.interaction_bwd(Z, w.grad_out[b][None].astype(np.float64), Zm)
        dZ, dZm = cache[b]
        k = np.searchsorted(uniq[pick], keys[o])
        g[k] += dZ[0, 1 + t]
        gm[k] += dZm[0, 1 + t]
    new, nm = orc.sparse_sgd(one, uniq[pick], g, gm, w.lr)
    got = host(fe.table[dev(uniq[pick])].float())
    # the row gradients carry the chain's error (bf16 operands, bf16-stored dZ, the tree)
    eg = step_bounds(int(np.diff(w.offsets).max()), w.dim, w.F, w.nnz, True,
                     fe.dZ.dtype == torch.bfloat16)["g"]
    assert_within(got, new, sgd_store_bound(new, gm, w.lr, eg, True), "Large updated rows",
                  mag=nm)


@pytest.mark.timeout(900)
def test_large_interaction_per_call_full_shape():
    """The matrix-core interaction at Large's full shape (32768 samples, F = 65, d = 128) on
    seeded inputs, forward and backward (dZ in fp32 and in bf16, as the step stores it):
    sampled samples against the oracle's bf16-operand mode, so only the fp32 accumulation
    (over d columns forward, F terms backward) and the bf16 store can differ."""
    B, F, d = 32768, 65, 128
    P = F * (F - 1) // 2
    rng = np.random.default_rng(31)
    Z = rng.standard_normal((B, F, d), dtype=np.float32)
    dR = rng.standard_normal((B, d + P), dtype=np.float32)
    say("Large-shape interaction, seeded inputs")
    Zd, dRd = dev(Z), dev(dR)
    R = host(ctr.ctr_dot_interaction_fwd(Zd, ctr.CTR_BF16))
    dZ32 = host(ctr.ctr_dot_interaction_bwd(Zd, dRd, ctr.CTR_BF16))
    dZb = torch.empty((B, F, d), dtype=torch.bfloat16, device=DEV)
    dZ16 = host(ctr.ctr_dot_interaction_bwd(Zd, dRd, ctr.CTR_BF16, dZ=dZb))
    del Zd, dRd, dZb
    samples = np.concatenate([[0, B - 1], rng.choice(B, size=30, replace=False)])
    Zs = Z[samples].astype(np.float64)
    want, mag = orc.interaction_fwd(Zs, bf16=True)
    assert_close(R[samples], want, mag, gamma(d), "Large-shape R")
    np.testing.assert_array_equal(R[samples, :d], Z[samples, 0])
    want, mag = orc.interaction_bwd(Zs, dR[samples].astype(np.float64), bf16=True)
    assert_close(dZ32[samples], want, mag, gamma(F), "Large-shape dZ fp32")
    assert_within(dZ16[samples], want, store_bound(want, mag, gamma(F), True),
                  "Large-shape dZ bf16", mag=mag)


@pytest.mark.timeout(900)
def test_large_sgd_hot_rows(large_run):
    """The fused backward + SGD as the step runs it at Large (bf16 gradient rows, bf16 table,
    nearest-even), at full size, with GPU-independent inputs: the table refilled from its
    definition, then one update from the generator's N(0,1) gradients (rounded to bf16 on the
    host) grouped by the step's own unique.  The 20 hottest rows (the deepest parts of the
    reduce-by-key tree, around 10^5 occurrences each) and random ones are checked against
    the oracle's update of the same rows.  Runs last: it overwrites the stepped table."""
    w, fe = large_run
    B, T, d = w.batch, w.num_tables, w.dim
    ctr.ctr_init_tables_hash(fe.table, w.rows, w.table_seed)
    rng = np.random.default_rng(6)
    dY = torch.from_numpy(rng.standard_normal((B, T, d), dtype=np.float32)).to(torch.bfloat16)
    dYd = dY.to(DEV)
    ctr.ctr_embbag_bwd_sgd(dYd, T * d, d, fe.offsets, B, T, w.nnz, fe.sorted_src, fe.num_unique,
                           fe.table, fe.uniq, w.lr, workspace=fe.ws_bwd)
    torch.cuda.synchronize()
    del dYd
    U = int(host(fe.num_unique)[0])
    uniq = host(fe.uniq[:U])
    keys = orc.form_keys(w.indices, w.offsets, T, B, w.row_base)
    counts = np.bincount(np.searchsorted(uniq, keys), minlength=U)
    pick = np.unique(np.concatenate([np.argsort(-counts)[:20], rng.choice(U, 200, replace=False)]))
    say("hot rows: most occurrences", int(counts[pick].max()))
    occ = np.flatnonzero(np.isin(keys, uniq[pick]))
    bag = np.searchsorted(w.offsets, occ, side="right") - 1
    sub_inv = np.searchsorted(uniq[pick], keys[occ]).astype(np.int32)
    dY64 = dY.float().numpy()
    sel = dY64[bag % B, bag // B].astype(np.float64)[:, None, :]
    g, gm = orc.embbag_bwd(sel, np.arange(occ.size + 1, dtype=np.int64), occ.size, 1, sub_inv,
                           pick.size)
    one = orc.Table(w.rows, w.dim, w.dtype, w.table_seed)
    new, nm = orc.sparse_sgd(one, uniq[pick], g, gm, w.lr)
    got = host(fe.table[dev(uniq[pick])].float())
    eg = gamma(segreduce_depth(w.nnz, d, True))
    assert_within(got, new, sgd_store_bound(new, gm, w.lr, eg, True), "Large hot rows updated",
                  mag=nm)
