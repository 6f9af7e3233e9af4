"""Property tests on the GPU over random small shapes (hypothesis, derandomized so every run
draws the same examples): each call of the path against the oracle, and a whole training
step on random little workloads.

Shapes are drawn across the kernels' boundaries: n from 0, keys over 1 to 62 bits and of
either sign, 1 to 4 tables with empty bags (up to 40 for the fused forward), every supported
row width, F from 2 up to past one 32-row MFMA block, batches that leave ragged blocks.  The bars are the parity bars: the
ID work bit-exact, floating point within rtol times the oracle's sum of |terms|.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import oracle as orc
from sparse_embedding_lookup_amd import ctr
from sparse_embedding_lookup_amd.pipeline import FrontEnd
from sparse_embedding_lookup_amd.workloads import Workload
from tests.chain import check_chain, oracle_dlrm_step
from tests.parity import assert_close, assert_within, gamma, pool_eps
from tests.test_gpu_parity import DEV, dev, gpu_table, host, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SETTINGS = settings(max_examples=20, deadline=None, derandomize=True, database=None,
                    suppress_health_check=list(HealthCheck))


@st.composite
def csr(draw, max_tables=4, max_batch=40, max_rows=500, max_len=10):
    T = draw(st.integers(1, max_tables))
    B = draw(st.integers(1, max_batch))
    rows = [draw(st.integers(1, max_rows)) for _ in range(T)]
    seed = draw(st.integers(0, 2 ** 31 - 1))
    empty = draw(st.sampled_from([0.0, 0.3]))
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, max_len + 1, size=(T, B))
    lengths[rng.random((T, B)) < empty] = 0
    off = np.zeros(T * B + 1, dtype=np.int64)
    off[1:] = np.cumsum(lengths.reshape(-1))
    ids = np.concatenate([rng.integers(0, rows[t], int(lengths[t].sum())) for t in range(T)])
    return T, B, rows, ids.astype(np.int64), off, seed


@SETTINGS
@given(n=st.integers(0, 2500), bits=st.integers(1, 62), signed=st.booleans(),
       modulus=st.sampled_from([0, 0, 7, 1000, 2 ** 31 - 1]), seed=st.integers(0, 2 ** 31 - 1))
def test_unique_flat_property(n, bits, signed, modulus, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, 1 << bits, size=n, dtype=np.int64)
    if signed:
        ids = np.where(rng.random(n) < 0.5, -ids, ids)
    keys = orc.form_keys(ids, np.array([0, n]), 1, 1, None, modulus)
    uniq, inv, nu, perm, seg = [host(x) for x in ctr.ctr_unique_ids(dev(ids), key_modulus=modulus)]
    ou, oi, op, os_ = orc.unique(keys)
    U = int(nu[0])
    assert U == ou.size
    np.testing.assert_array_equal(uniq[:U], ou)
    np.testing.assert_array_equal(inv[:n], oi)
    np.testing.assert_array_equal(perm[:n], op)
    np.testing.assert_array_equal(seg[:U + 1], os_)


@SETTINGS
@given(c=csr())
def test_unique_tables_property(c):
    T, B, rows, ids, off, _ = c
    rb = np.zeros(T + 1, dtype=np.int64)
    rb[1:] = np.cumsum(rows)
    keys = orc.form_keys(ids, off, T, B, rb)
    res = ctr.ctr_unique_ids(dev(ids), offsets=dev(off), batch=B, num_tables=T, row_base=dev(rb),
                             total_rows=int(rb[-1]))
    uniq, inv, nu, perm, seg = [host(x) for x in res]
    ou, oi, op, os_ = orc.unique(keys)
    U = int(nu[0])
    n = ids.size
    assert U == ou.size
    np.testing.assert_array_equal(uniq[:U], ou)
    np.testing.assert_array_equal(inv[:n], oi)
    np.testing.assert_array_equal(perm[:n], op)
    np.testing.assert_array_equal(seg[:U + 1], os_)


@SETTINGS
@given(c=csr(), dtype=st.sampled_from(["f32", "bf16"]), wide=st.integers(0, 4))
def test_embbag_fwd_property(c, dtype, wide):
    T, B, rows, ids, off, seed = c
    dim = [4, 8, 16, 32, 64][wide] * (2 if dtype == "bf16" else 1)
    say("embbag_fwd property", T, B, rows, dtype, dim, ids.size)
    t = gpu_table(rows, dim, dtype, seed % 1000)
    tab = orc.Table(rows, dim, dtype, seed % 1000)
    out = torch.full((B, T, dim), float("nan"), device=DEV)
    ctr.ctr_embbag_fwd(t, dev(ids), dev(off), B, T, out, T * dim, dim, row_base=dev(tab.row_base))
    want, mag = orc.embbag_fwd(tab, ids, off, B)
    assert_within(host(out), want, pool_eps(off, B, T) * mag, "embbag_fwd property", mag=mag)


@SETTINGS
@given(B=st.integers(1, 40), F=st.integers(2, 40), compute=st.sampled_from(["f32", "bf16"]),
       wide=st.integers(0, 3), seed=st.integers(0, 2 ** 31 - 1))
def test_interaction_property(B, F, compute, wide, seed):
    d = [4, 16, 32, 64][wide] if compute == "f32" else [16, 32, 64, 128][wide]
    say("interaction property", B, F, compute, d)
    rng = np.random.default_rng(seed)
    Z = rng.standard_normal((B, F, d)).astype(np.float32)
    dR = rng.standard_normal((B, d + F * (F - 1) // 2)).astype(np.float32)
    code = ctr.CTR_BF16 if compute == "bf16" else ctr.CTR_F32
    bf = compute == "bf16"
    R = host(ctr.ctr_dot_interaction_fwd(dev(Z), code))
    want, mag = orc.interaction_fwd(Z.astype(np.float64), bf16=bf)
    assert_close(R, want, mag, gamma(d), "interaction fwd property")
    dZ = host(ctr.ctr_dot_interaction_bwd(dev(Z), dev(dR), code))
    want, mag = orc.interaction_bwd(Z.astype(np.float64), dR.astype(np.float64), bf16=bf)
    assert_close(dZ, want, mag, gamma(F), "interaction bwd property")


@settings(max_examples=12, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
@given(c=csr(max_tables=3, max_batch=30, max_rows=300, max_len=8),
       dtype=st.sampled_from(["f32", "bf16"]), wide=st.integers(0, 2))
def test_whole_step_property(c, dtype, wide):
    """One serial training step (pooling, interaction, its backward, unique, fused backward
    and SGD) on a random little workload, against the oracle's chain."""
    T, B, rows, ids, off, seed = c
    dim = [16, 32, 64][wide]
    rng = np.random.default_rng(seed + 1)
    F = T + 1
    P = F * (F - 1) // 2
    w = Workload("property", T, rows, dim, dtype, B, ids, off,
                 rng.standard_normal((B, dim)).astype(np.float32),
                 rng.standard_normal((B, dim + P)).astype(np.float32), 0.01, dtype,
                 table_seed=seed % 1000)
    say("whole step property", T, B, rows, dtype, dim, ids.size)
    fe = FrontEnd(w, DEV, keep_grads=True)
    before = host(fe.table.float())
    fe.step()
    o = oracle_dlrm_step(w)
    check_chain(w, fe, o)
    tbl = host(fe.table.float())
    untouched = np.ones(sum(rows), bool)
    untouched[o["uniq"]] = False
    np.testing.assert_array_equal(tbl[untouched], before[untouched])


@SETTINGS
@given(T=st.integers(1, 40), B=st.integers(1, 300), tdt=st.sampled_from(["f32", "bf16"]),
       compute=st.sampled_from(["f32", "bf16"]), wide=st.integers(0, 3),
       empty=st.sampled_from([0.0, 0.3]), max_len=st.integers(1, 12),
       seed=st.integers(0, 2 ** 31 - 1))
def test_fused_forward_property(T, B, tdt, compute, wide, empty, max_len, seed):
    """ctr_embbag_interaction_fwd on random shapes: Z's pooled rows against the oracle's
    pooling, R against the oracle's interaction of the kernel's own Z."""
    dim = [16, 32, 64, 128][wide]
    F = T + 1
    if compute == "bf16" and F > 128:
        return
    per = F * (dim + 8) * 2 if compute == "bf16" else F * (dim + 1) * 4
    if per > 47104:                       # one sample's copy beyond what one block holds
        return
    say("fused forward property", T, B, tdt, compute, dim, empty, max_len)
    rng = np.random.default_rng(seed)
    rows = [int(r) for r in rng.integers(1, 400, size=T)]
    lengths = rng.integers(1, max_len + 1, size=(T, B))
    lengths[rng.random((T, B)) < empty] = 0
    off = np.zeros(T * B + 1, dtype=np.int64)
    off[1:] = np.cumsum(lengths.reshape(-1))
    ids = np.concatenate([rng.integers(0, rows[t], int(lengths[t].sum())) for t in range(T)])
    ids = ids.astype(np.int64)
    t = gpu_table(rows, dim, tdt, seed % 1000)
    tab = orc.Table(rows, dim, tdt, seed % 1000)
    dense = rng.standard_normal((B, dim)).astype(np.float32)
    Z = torch.full((B, F, dim), float("nan"), device=DEV)
    Z[:, 0, :] = dev(dense)
    code = ctr.CTR_BF16 if compute == "bf16" else ctr.CTR_F32
    R = ctr.ctr_embbag_interaction_fwd(t, dev(ids), dev(off), Z, code,
                                       row_base=dev(tab.row_base))
    Zg, Rg = host(Z), host(R)
    want, mag = orc.embbag_fwd(tab, ids, off, B)
    assert_within(Zg[:, 1:], want, pool_eps(off, B, T) * mag, "fused Z property", mag=mag)
    np.testing.assert_array_equal(Rg[:, :dim], dense)
    want, mag = orc.interaction_fwd(Zg.astype(np.float64), bf16=compute == "bf16")
    assert_close(Rg, want, mag, gamma(dim), "fused R property")
