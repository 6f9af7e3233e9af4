"""One front-end training step end to end against the oracle's own chain (pooling, the
pairwise-dot interaction, its gradient, unique, the per-row gradient sums and the SGD
update), each output within the bound its chain of roundings gives (tests/parity.py)."""
import numpy as np
import torch

from oracle import oracle as orc
from tests.parity import (assert_close, assert_within, pool_eps, sgd_store_bound, step_bounds,
                          store_bound)


def host(t):
    torch.cuda.synchronize()
    if t.dtype in (torch.bfloat16, torch.float16):   # widen (exact); numpy has no bfloat16
        t = t.float()
    return t.detach().cpu().numpy()


def oracle_dlrm_step(w):
    tab = orc.Table(w.rows, w.dim, w.dtype, w.table_seed)
    pooled, pmag = orc.embbag_fwd(tab, w.indices, w.offsets, w.batch)
    B, F, d = w.batch, w.F, w.dim
    Z = np.empty((B, F, d))
    Zm = np.empty((B, F, d))
    Z[:, 0] = w.dense
    Zm[:, 0] = np.abs(w.dense)
    Z[:, 1:] = pooled
    Zm[:, 1:] = pmag
    R, Rm = orc.interaction_fwd(Z, Zm)
    dZ, dZm = orc.interaction_bwd(Z, w.grad_out.astype(np.float64), Zm)
    keys = orc.form_keys(w.indices, w.offsets, w.num_tables, B, w.row_base)
    uniq, inv, perm, seg = orc.unique(keys)
    g, gm = orc.embbag_bwd(dZ[:, 1:], w.offsets, B, w.num_tables, inv, uniq.size, dZm[:, 1:])
    new, nm = orc.sparse_sgd(tab, uniq, g, gm, w.lr)
    return dict(Z=Z, Zm=Zm, R=R, Rm=Rm, dZ=dZ, dZm=dZm, keys=keys, uniq=uniq, inv=inv,
                perm=perm, g=g, gm=gm, new=new, nm=nm)


def check_chain(w, fe, o, table_rows=True):
    """fe (a FrontEnd after one step) against o (oracle_dlrm_step of the same workload):
    pooled Z, R, dZ, the row gradients and the updated rows within step_bounds; the dense
    slot of Z, unique keys and the inverse map bit for bit."""
    grad_bf16 = fe.dZ.dtype == torch.bfloat16
    eb = step_bounds(int(np.diff(w.offsets).max()) if w.nnz else 0, w.dim, w.F, w.nnz,
                     w.compute == "bf16", grad_bf16)
    Zg = host(fe.Z)
    np.testing.assert_array_equal(Zg[:, 0], w.dense)
    assert_within(Zg[:, 1:], o["Z"][:, 1:],
                  pool_eps(w.offsets, w.batch, w.num_tables) * o["Zm"][:, 1:], "Z",
                  mag=o["Zm"][:, 1:])
    assert_close(host(fe.R), o["R"], o["Rm"], eb["R"], "R")
    assert_within(host(fe.dZ), o["dZ"], store_bound(o["dZ"], o["dZm"], eb["dZ"], grad_bf16),
                  "dZ", mag=o["dZm"])
    U = int(host(fe.num_unique)[0])
    assert U == o["uniq"].size
    np.testing.assert_array_equal(host(fe.uniq)[:U], o["uniq"])
    np.testing.assert_array_equal(host(fe.inverse)[:w.nnz], o["inv"])
    assert_close(host(fe.row_grads)[:U], o["g"], o["gm"], eb["g"], "row grads")
    if table_rows:
        rows = torch.from_numpy(np.ascontiguousarray(o["uniq"])).to(fe.table.device)
        tbl = host(fe.table[rows].float())
        assert_within(tbl, o["new"], sgd_store_bound(o["new"], o["gm"], w.lr, eb["g"], w.dtype),
                      "updated rows", mag=o["nm"])
    return eb
