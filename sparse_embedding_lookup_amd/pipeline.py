"""One training step of the sparse front end, as a chain of libctr calls.

Nothing here computes: torch allocates device buffers and uploads the batch, and every step
of the path (keys, unique, pooling, interaction, gradients, update) is a C-ABI call.

DLRM-shaped step (tables + dense vector, "Meta DLRM" 02 and "DHEN" notes 2.1 / 3.1):
  forward   ctr_embbag_fwd writes the pooled vectors straight into Z[:, 1:, :] (the dense
            vector sits in Z[:, 0, :] since the batch upload), ctr_dot_interaction_fwd -> R
  backward  ctr_dot_interaction_bwd -> dZ, ctr_unique_ids over the batch's rows,
            ctr_embbag_bwd(dZ[:, 1:, :]) -> per-row gradients, ctr_sparse_sgd.
TensorNet-shaped step ("How TensorNet Supercharges ...", "Core Optimizations"):
  ctr_unique_ids(ids mod rows) -> contiguous indices, ctr_gather_rows -> batch-sized matrix
  E, ctr_embbag_fwd(E, indices = inverse) -> per-slot vectors; backward ctr_embbag_bwd over
  the same segments, ctr_sparse_sgd on the table.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import ctr
from .workloads import Workload


def _dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class FrontEnd:
    """Device state for one workload: the tables, the batch and every buffer of the path."""

    def __init__(self, w: Workload, device="cuda", table: Optional[torch.Tensor] = None):
        self.w = w
        self.device = torch.device(device)
        self.bf16 = w.dtype == "bf16"
        self.compute = ctr.CTR_BF16 if w.compute == "bf16" else ctr.CTR_F32
        tdt = torch.bfloat16 if self.bf16 else torch.float32
        if table is None:
            table = torch.empty((w.total_rows, w.dim), dtype=tdt, device=self.device)
            ctr.ctr_init_table_hash(table, w.rows, w.table_seed)
        self.table = table
        self.row_base = _dev(w.row_base, self.device)
        self.indices = _dev(w.indices, self.device)
        self.offsets = _dev(w.offsets, self.device)
        self.nnz = w.nnz
        B, T, d = w.batch, w.num_tables, w.dim
        if w.interaction:
            F = w.F
            self.Z = torch.empty((B, F, d), dtype=torch.float32, device=self.device)
            self.Z[:, 0, :].copy_(_dev(w.dense, self.device))        # batch upload
            self.R = torch.empty((B, d + w.P), dtype=torch.float32, device=self.device)
            self.dR = _dev(w.grad_out, self.device)
            self.dZ = torch.empty_like(self.Z)
        else:
            n = w.nnz
            self.E = torch.empty((max(n, 1), d), dtype=torch.float32, device=self.device)
            self.out = torch.empty((max(n, 1), d), dtype=torch.float32, device=self.device)
            self.dout = _dev(w.grad_out.reshape(n, d), self.device)
        self.row_grads = torch.empty((max(self.nnz, 1), d), dtype=torch.float32,
                                     device=self.device)
        n = self.nnz
        dv = self.device
        self.ws_unique = torch.empty(max(ctr.unique_workspace_bytes(n), 256), dtype=torch.uint8,
                                     device=dv)
        self.ws_bwd = torch.empty(max(ctr.embbag_bwd_workspace_bytes(n, d), 256),
                                  dtype=torch.uint8, device=dv)
        self.uniq = torch.empty(max(n, 1), dtype=torch.int64, device=dv)
        self.inverse = torch.empty(max(n, 1), dtype=torch.int32, device=dv)
        self.num_unique = torch.zeros(1, dtype=torch.int32, device=dv)
        self.perm = torch.empty(max(n, 1), dtype=torch.int32, device=dv)
        self.seg = torch.empty(n + 1, dtype=torch.int32, device=dv)
        self._unique_out = (self.uniq, self.inverse, self.num_unique, self.perm, self.seg)
        self.side = None

    # ------------------------------------------------------------------ steps of the path
    def unique(self):
        w = self.w
        if w.interaction:
            ctr.ctr_unique_ids(self.indices, offsets=self.offsets, batch=w.batch,
                               num_tables=w.num_tables, row_base=self.row_base,
                               total_rows=w.total_rows, workspace=self.ws_unique,
                               out=self._unique_out)
        else:
            ctr.ctr_unique_ids(self.indices, key_modulus=w.key_modulus, workspace=self.ws_unique,
                               out=self._unique_out)

    def _embbag_fwd(self):
        w = self.w
        if w.interaction:
            F, d = w.F, w.dim
            ctr.ctr_embbag_fwd(self.table, self.indices, self.offsets, w.batch, w.num_tables,
                               self.Z[:, 1:, :], F * d, d, row_base=self.row_base)
        else:
            ctr.ctr_embbag_fwd(self.E, self.inverse, self.offsets, self.nnz, 1, self.out,
                               w.dim, 0)

    def _gather_rows(self):
        ctr.ctr_gather_rows(self.table, self.uniq, self.num_unique, self.nnz, out=self.E)

    def _interaction_fwd(self):
        ctr.ctr_dot_interaction_fwd(self.Z, self.compute, self.R)

    def _interaction_bwd(self):
        ctr.ctr_dot_interaction_bwd(self.Z, self.dR, self.compute, self.dZ)

    def _embbag_bwd(self):
        w = self.w
        d = w.dim
        perm = self.perm[:self.nnz]
        if w.interaction:
            F = w.F
            ctr.ctr_embbag_bwd(self.dZ[:, 1:, :], F * d, d, self.offsets, w.batch,
                               w.num_tables, d, perm, self.inverse, self.num_unique,
                               self.row_grads, workspace=self.ws_bwd)
        else:
            ctr.ctr_embbag_bwd(self.dout, d, 0, self.offsets, self.nnz, 1, d, perm,
                               self.inverse, self.num_unique, self.row_grads,
                               workspace=self.ws_bwd)

    def _sparse_sgd(self):
        ctr.ctr_sparse_sgd(self.table, self.uniq, self.num_unique, self.nnz, self.row_grads,
                           self.w.lr)

    def stages(self):
        """The step's calls in dependency order, as (name, fn)."""
        if self.w.interaction:
            return [("embbag_fwd", self._embbag_fwd), ("interaction_fwd", self._interaction_fwd),
                    ("interaction_bwd", self._interaction_bwd), ("unique", self.unique),
                    ("embbag_bwd", self._embbag_bwd), ("sparse_sgd", self._sparse_sgd)]
        return [("unique", self.unique), ("gather_rows", self._gather_rows),
                ("embbag_fwd", self._embbag_fwd), ("embbag_bwd", self._embbag_bwd),
                ("sparse_sgd", self._sparse_sgd)]

    def forward(self):
        if self.w.interaction:
            self._embbag_fwd()
            self._interaction_fwd()
        else:
            self.unique()
            self._gather_rows()
            self._embbag_fwd()

    def backward(self):
        if self.w.interaction:
            self._interaction_bwd()
            self.unique()
        self._embbag_bwd()
        self._sparse_sgd()

    def step(self, mark=None):
        """One training step.  With tables and a dense vector, the batch's unique runs on a
        second stream (default priority) beside the forward and the interaction gradient,
        which do not need it.  ``mark(name, fn)`` may wrap a stage (e.g. with events on the
        stream it runs on); by default it just calls it."""
        run = mark if mark is not None else (lambda name, fn: fn())
        if not self.w.interaction:
            for name, fn in self.stages():
                run(name, fn)
            return
        main = torch.cuda.current_stream(self.device)
        if self.side is None:
            self.side = torch.cuda.Stream(device=self.device)
        self.side.wait_stream(main)
        with torch.cuda.stream(self.side):
            run("unique", self.unique)
        run("embbag_fwd", self._embbag_fwd)
        run("interaction_fwd", self._interaction_fwd)
        run("interaction_bwd", self._interaction_bwd)
        main.wait_stream(self.side)
        run("embbag_bwd", self._embbag_bwd)
        run("sparse_sgd", self._sparse_sgd)
