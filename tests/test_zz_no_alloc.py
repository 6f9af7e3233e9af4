"""ctr_embbag_bwd_sgd_noalloc (the backward + SGD entry that allocates nothing: its carries
live in the library's per-GPU scratch array) against ctr_embbag_bwd_sgd (same kernels,
caller workspace): bit-identical row sums and updated tables, on consecutive calls that
reuse the scratch, the later ones with smaller inputs."""
import sys

import numpy as np
import pytest
import torch

from sparse_embedding_lookup_amd import ctr, workloads
from sparse_embedding_lookup_amd.pipeline import FrontEnd

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _pair(w, seed, grad_dtype, with_table, rows=False):
    """One call of each entry on the same unique, gradients and starting table.  rows: the
    unique's 8-byte row entries (CTR_SRC_ROWS), which serve the update without row sums."""
    fe = FrontEnd(w, DEV, src_rows=rows)
    fe.unique()
    B, T, d, n = w.batch, w.num_tables, w.dim, w.nnz
    need = ctr.noalloc_scratch_bytes(n, d)
    say("noalloc", w.name, "B", B, "nnz", n, "scratch bytes", need, "of",
        ctr.noalloc_scratch_capacity())
    assert need <= ctr.noalloc_scratch_capacity()
    gen = torch.Generator(device=DEV).manual_seed(seed)
    g = torch.randn((B, T + 1, d), generator=gen, device=DEV).to(grad_dtype)
    U = int(fe.num_unique.cpu()[0])
    ra = torch.full((n, d), float("nan"), device=DEV)
    rb = torch.full((n, d), float("nan"), device=DEV)
    if with_table:
        ta, tb = fe.table.clone(), fe.table.clone()
        ctr.ctr_embbag_bwd_sgd(g[:, 1:, :], (T + 1) * d, d, fe.offsets, B, T, n, fe.sorted_src,
                               fe.num_unique, ta, fe.uniq, w.lr,
                               row_grads=None if rows else ra)
        ctr.ctr_embbag_bwd_sgd_noalloc(g[:, 1:, :], (T + 1) * d, d, fe.offsets, B, T, n,
                                       fe.sorted_src, fe.num_unique, tb, fe.uniq, w.lr,
                                       row_grads=None if rows else rb)
        torch.cuda.synchronize()
        assert torch.equal(ta, tb), "updated tables differ"
        assert not torch.equal(ta, fe.table), "the update changed nothing"
        if rows:
            return
    else:
        ctr.ctr_embbag_bwd(g[:, 1:, :], (T + 1) * d, d, fe.offsets, B, T, d, None, None,
                           fe.num_unique, row_grads=ra, sorted_src=fe.sorted_src, nnz=n)
        ctr.ctr_embbag_bwd_sgd_noalloc(g[:, 1:, :], (T + 1) * d, d, fe.offsets, B, T, n,
                                       fe.sorted_src, fe.num_unique, None, None, w.lr,
                                       row_grads=rb, dim=d)
        torch.cuda.synchronize()
    assert torch.isfinite(ra[:U]).all()
    assert torch.equal(ra[:U], rb[:U]), "row sums differ"


def test_noalloc_matches_workspace_entry_on_consecutive_calls():
    # bf16 table and bf16 gradient rows (the matrix-core step's backward), then a smaller
    # fp32 batch, then row sums alone: each call reuses the scratch the previous one left
    _pair(workloads.criteo(batch=1024), 1, torch.bfloat16, True)
    _pair(workloads.small(batch=256), 2, torch.float32, True)
    _pair(workloads.small(batch=64), 3, torch.float32, False)
    # the same through row entries (no row sums): a bf16 batch, then a smaller fp32 one
    _pair(workloads.criteo(batch=512), 4, torch.bfloat16, True, rows=True)
    _pair(workloads.small(batch=128), 5, torch.float32, True, rows=True)


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    w = workloads.small(batch=64)
    fe = FrontEnd(w, DEV)
    fe.unique()
    n_big = 1 << 26                           # claims 67M occurrences of 64-wide rows
    assert ctr.noalloc_scratch_bytes(n_big, w.dim) > ctr.noalloc_scratch_capacity()
    g = torch.zeros((w.batch, w.num_tables + 1, w.dim), device=DEV)
    before = fe.table.clone()
    with pytest.raises(ctr.CtrError) as e:
        ctr.ctr_embbag_bwd_sgd_noalloc(g[:, 1:, :], (w.num_tables + 1) * w.dim, w.dim,
                                       fe.offsets, w.batch, w.num_tables, n_big, fe.sorted_src,
                                       fe.num_unique, fe.table, fe.uniq, w.lr)
    assert "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(before, fe.table)      # rejected before any launch
