"""A whole DLRM training step on the GPU ("Meta DLRM", 02: bottom MLP, embeddings, pairwise
dots, top MLP, sigmoid; "DHEN" notes, 7.1: normalized entropy), checked against the oracle
stage by stage on the GPU's own stage inputs.

Each stage's output is recomputed by the oracle from the values the GPU handed to it (the
previous stage's GPU output and the parameters as they were before the step), so the check
covers both every call and the wiring between calls: which buffer feeds which layer, that
the top MLP's input gradient is the interaction's dR, that dZ[:, 0, :] feeds the bottom
MLP, and that every parameter moves by its own gradient.  Dense-layer and head stages use
rtol = 1e-5 (identical operand rounding on both sides); the interaction stages use the
interaction's bar for the workload's compute type.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from sparse_embedding_lookup_amd import workloads
from sparse_embedding_lookup_amd.dlrm import DlrmStep
from tests.parity import (RTOL_F32, assert_close, assert_within, gamma, pool_eps, segreduce_depth,
                          sgd_store_bound, store_bound)
from tests.test_gpu_parity import DEV, host, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

WORKLOADS = {"tiny": workloads.tiny, "small_b256": lambda: workloads.small(batch=256),
             "criteo_b128": lambda: workloads.criteo(batch=128)}


def _f32(t):
    return host(t.float()) if t.dtype == torch.bfloat16 else host(t)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_dlrm_step_stage_by_stage(name):
    w = WORKLOADS[name]()
    inp = workloads.dlrm_inputs(w, seed=1)
    say("dlrm step", name, w.batch, w.F, w.dim, w.compute)
    s = DlrmStep(w, inp, DEV)
    bf16 = w.compute == "bf16"
    layers = s.bottom + s.top
    before = [(host(L.W), host(L.b)) for L in layers]
    s.step()
    torch.cuda.synchronize()
    nb = len(s.bottom)

    # forward: bottom MLP on the continuous features, its output in Z[:, 0, :]
    x = inp.dense_raw
    for i, L in enumerate(s.bottom):
        want, mag = orc.dense_fwd(x, before[i][0], before[i][1], True, bf16)
        x = host(s.b_out[i])
        assert_close(x, want, mag, RTOL_F32, "bottom layer %d" % i)
    Z = host(s.fe.Z)
    np.testing.assert_array_equal(Z[:, 0, :], x)
    # pooled rows (the fused forward by default for matrix-core dots, else the two calls)
    assert s.fe.fused_fwd == (bf16 and w.F <= 32)
    pooled, pmag = orc.embbag_fwd(orc.Table(w.rows, w.dim, w.dtype, w.table_seed), w.indices,
                                  w.offsets, w.batch)
    assert_within(Z[:, 1:, :], pooled, pool_eps(w.offsets, w.batch, w.num_tables) * pmag,
                  "pooled", mag=pmag)
    # the interaction on the GPU's Z: matrix-core dots take the same bf16 operands as the
    # oracle's bf16 mode, so only the fp32 accumulation over d columns differs
    R, Rm = orc.interaction_fwd(Z.astype(np.float64), bf16=bf16)
    Rg = host(s.fe.R)
    assert_close(Rg, R, Rm, gamma(w.dim), "R")
    # top MLP on the GPU's R, then the head on its logits
    x = Rg
    for i, L in enumerate(s.top):
        j = nb + i
        want, mag = orc.dense_fwd(x, before[j][0], before[j][1], L.relu, bf16)
        x = host(s.t_out[i])
        assert_close(x, want, mag, RTOL_F32, "top layer %d" % i)
    prob, dl, dlm, st, stm = orc.logistic_ne(x[:, 0], inp.labels)
    assert_close(host(s.dlogits)[:, 0], dl, dlm + 1e-30, RTOL_F32, "d logits")
    got = host(s.stats).astype(np.float64)
    assert_close(got, st, stm, RTOL_F32, "head stats")
    assert 0.3 < got[2] < 5.0                         # an untrained model: NE near 1

    # backward through the top MLP: each layer's dX is the next-lower layer's dY; the first
    # layer's dX is the interaction's dR
    dY = host(s.dlogits)
    t_in = [Rg] + [host(t) for t in s.t_out[:-1]]
    for i in reversed(range(len(s.top))):
        L, j = s.top[i], nb + i
        o = orc.dense_bwd_sgd(t_in[i], before[j][0], before[j][1], L.relu, host(s.t_out[i]), dY,
                              bf16, np.float32(s.lr))
        assert_close(host(L.W), o["W"], o["Wm"], RTOL_F32, "top W %d" % i)
        assert_close(host(L.b), o["b"], o["bm"], RTOL_F32, "top b %d" % i)
        dY = host(s.t_dx[i])
        assert_close(dY, o["dX"], o["dXm"], RTOL_F32, "top dX %d" % i)
    np.testing.assert_array_equal(host(s.fe.dR), dY)

    # interaction backward on the GPU's dR
    dZ, dZm = orc.interaction_bwd(Z.astype(np.float64), dY.astype(np.float64), bf16=bf16)
    dZg = _f32(s.fe.dZ)
    assert_within(dZg, dZ, store_bound(dZ, dZm, gamma(w.F), s.fe.dZ.dtype == torch.bfloat16),
                  "dZ", mag=dZm)

    # embedding rows: the touched rows move by their summed gradient from the GPU's dZ
    tab = orc.Table(w.rows, w.dim, w.dtype, w.table_seed)
    keys = orc.form_keys(w.indices, w.offsets, w.num_tables, w.batch, w.row_base)
    uniq, inv, _, _ = orc.unique(keys)
    g, gm = orc.embbag_bwd(dZg[:, 1:].astype(np.float64), w.offsets, w.batch, w.num_tables, inv,
                           uniq.size)
    new, nm = orc.sparse_sgd(tab, uniq, g, gm, w.lr)
    rows = _f32(s.fe.table)[uniq]
    eg = gamma(segreduce_depth(w.nnz, w.dim, s.fe.dZ.dtype == torch.bfloat16))
    assert_within(rows, new, sgd_store_bound(new, gm, w.lr, eg, w.dtype), "table rows",
                  mag=nm)

    # backward through the bottom MLP, starting from dZ[:, 0, :]
    dY = dZg[:, 0, :]
    b_in = [inp.dense_raw] + [host(t) for t in s.b_out[:-1]]
    for i in reversed(range(nb)):
        L = s.bottom[i]
        o = orc.dense_bwd_sgd(b_in[i], before[i][0], before[i][1], True, host(s.b_out[i]), dY,
                              bf16, np.float32(s.lr), want_dx=i > 0)
        assert_close(host(L.W), o["W"], o["Wm"], RTOL_F32, "bottom W %d" % i)
        assert_close(host(L.b), o["b"], o["bm"], RTOL_F32, "bottom b %d" % i)
        if i > 0:
            dY = host(s.b_dx[i])
            assert_close(dY, o["dX"], o["dXm"], RTOL_F32, "bottom dX %d" % i)


@pytest.mark.parametrize("name", ["small_b256", "criteo_b128"])
def test_dlrm_graph_replay_matches_eager_steps(name):
    """A one-step HIP graph replayed three times, with eager work and a synchronize between
    replays, leaves every parameter, the table and the head's statistics bit-identical to
    eager steps after every replay (the dense calls allocate nothing and keep no state)."""
    w = WORKLOADS[name]()
    inp = workloads.dlrm_inputs(w, seed=2)
    a = DlrmStep(w, inp, DEV)
    b = DlrmStep(w, inp, DEV)
    g = b.capture(steps=1)
    for k in range(3):
        a.step()
        g.replay()
        torch.cuda.synchronize()
        for pa, pb in zip(a.parameters(), b.parameters()):
            assert torch.equal(pa, pb), k
        assert torch.equal(a.fe.table, b.fe.table), k
        assert torch.equal(a.stats, b.stats), k


def test_dlrm_training_lowers_the_loss():
    """Repeated steps on one batch lower its cross-entropy (a sanity check of the update
    signs through every stage)."""
    w = workloads.small(batch=512)
    inp = workloads.dlrm_inputs(w, seed=3)
    s = DlrmStep(w, inp, DEV, lr=0.05)
    s.step()
    first = float(host(s.stats)[0])
    for _ in range(30):
        s.step()
    last = float(host(s.stats)[0])
    assert last < 0.9 * first, (first, last)


@pytest.mark.parametrize("graph", [False, True])
@pytest.mark.parametrize("unique_at", ["start", "after_pool"])
def test_dlrm_overlapped_unique_matches_serial(graph, unique_at):
    """The unique on a side stream (overlap=True), forked when the step starts or after the
    pooling, gives the same bits as running it in line, step after step, eager or replayed
    from a graph."""
    w = workloads.criteo(batch=128)
    inp = workloads.dlrm_inputs(w, seed=4)
    a = DlrmStep(w, inp, DEV, overlap=False)
    b = DlrmStep(w, inp, DEV, overlap=True, unique_at=unique_at)
    g = b.capture(steps=1) if graph else None
    for k in range(3):
        a.step()
        if graph:
            g.replay()
        else:
            b.step()
        torch.cuda.synchronize()
        for pa, pb in zip(a.parameters(), b.parameters()):
            assert torch.equal(pa, pb), k
        assert torch.equal(a.fe.table, b.fe.table), k
        assert torch.equal(a.stats, b.stats), k
