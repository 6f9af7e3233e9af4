"""A whole DLRM training step around the sparse front end, as a chain of libctr calls.

"Meta DLRM" (upskillscore.com), 02 "Arquitetura": the continuous features pass through a
bottom MLP whose output is the dense vector of the interaction, the categorical features
through the embedding tables; the pairwise dots of all those vectors, concatenated with the
dense vector, pass through a top MLP and a sigmoid that gives the click probability.
"DHEN" notes, 7.1 "Setup": the loss is normalized entropy (the mean cross-entropy over the
entropy of the batch's click rate); training follows the gradient of the mean
cross-entropy, NE's numerator (the denominator does not depend on the parameters).

Forward   bottom layers (ReLU each; the last writes Z[:, 0, :]), pooled bags into
          Z[:, 1:, :], the interaction -> R, top layers (ReLU, then a linear logit), the head
          (sigmoid, cross-entropy sums, NE, d logit).
Backward  top layers in reverse (each updates its W, b by SGD; the first writes dR), the
          interaction backward -> dZ, the fused embedding backward with the sparse SGD step,
          bottom layers in reverse (dZ[:, 0, :] feeds the last).
The batch's unique needs only its IDs: with overlap=True it runs on a side stream from the
step's start (after everything before the step) and is joined just before the embedding
backward, so it overlaps the forward, the top MLP's backward and the interaction's.  The
bottom MLP's backward then takes the side stream beside the embedding backward.
Nothing here computes: torch allocates, and every step is a C-ABI call marshalled once.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

from . import ctr
from .pipeline import FrontEnd, _dev
from .workloads import DlrmInputs, Workload


class _Layer:
    """One fully connected layer: parameters, its output buffer and its input's gradient."""

    def __init__(self, W: np.ndarray, b: np.ndarray, relu: bool, device):
        self.W = _dev(W, device)
        self.b = _dev(b, device)
        self.relu = relu
        self.N, self.K = W.shape


class DlrmStep:
    """Device state of a DLRM training step: the front end (tables, batch, Z, R, dR, dZ) and
    the two MLPs.  MLP arithmetic follows the workload's interaction compute type (fp32, or
    bf16 operands with fp32 accumulation)."""

    def __init__(self, w: Workload, inputs: DlrmInputs, device="cuda",
                 table: Optional[torch.Tensor] = None, lr: Optional[float] = None,
                 overlap: bool = True, fused_fwd: Optional[bool] = None,
                 unique_at: str = "start"):
        assert w.interaction, "the DLRM step needs the pooled-interaction workload"
        self.w = w
        self.device = torch.device(device)
        self.overlap = overlap
        # with overlap, where the batch's unique forks to the side stream: "start" (before
        # the bottom MLP) or "after_pool" (after the pooling, so the sort overlaps the
        # interaction and the MLPs instead of the HBM-bound gathers)
        assert unique_at in ("start", "after_pool")
        self.unique_at = unique_at
        self.side = torch.cuda.Stream(device=self.device) if overlap else None
        # R padded to 16-byte rows: the top MLP's first layer reads it with vector loads
        # fused forward (pooling and interaction in one call) by default where the dots run
        # on matrix cores and a sample's vectors fit one 32-row tile (F <= 32): the Criteo-
        # shaped step 1.278 -> 1.265 ms.  With 65 vectors (Large) a fused block gathers from
        # every table at once while the batch's sort runs beside it: 15.08 -> 15.32 ms, so
        # the two calls stay; with fp32 dots (Small) the two forms are level.
        if fused_fwd is None:
            fused_fwd = w.compute == "bf16" and w.F <= 32
        self.fe = FrontEnd(w, device, table=table, pad_r=True, fused_fwd=fused_fwd)
        self.lr = float(w.lr if lr is None else lr)
        self.compute = self.fe.compute
        dv = self.device
        B, F, d = w.batch, w.F, w.dim
        self.dense_raw = _dev(inputs.dense_raw, dv)
        self.labels = _dev(inputs.labels, dv)
        self.bottom = [_Layer(W, b, True, dv) for W, b in inputs.bottom]
        nt = len(inputs.top)
        self.top = [_Layer(W, b, i < nt - 1, dv) for i, (W, b) in enumerate(inputs.top)]
        assert self.bottom[-1].N == d and self.top[0].K == d + w.P and self.top[-1].N == 1
        # activations: the bottom MLP's last output is Z[:, 0, :]; the top's last the logits
        zs = self.fe.Z[:, 0, :]
        self.b_out = [torch.empty((B, L.N), device=dv) for L in self.bottom[:-1]] + [zs]
        self.t_out = [torch.empty((B, L.N), device=dv) for L in self.top]
        self.logits = self.t_out[-1]
        self.dlogits = torch.empty((B, 1), device=dv)
        self.prob = torch.empty(B, device=dv)
        self.stats = torch.zeros(3, device=dv)
        # gradients of each layer's input (top: the first writes the front end's dR)
        self.t_dx = [self.fe.dR] + [torch.empty((B, L.K), device=dv) for L in self.top[1:]]
        self.b_dx = [None] + [torch.empty((B, L.K), device=dv) for L in self.bottom[1:]]
        ws = max(ctr.dense_bwd_workspace_bytes(B, L.K, L.N, True, L.relu, self.compute)
                 for L in self.bottom + self.top)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dv)
        self._prepare()

    def _prepare(self):
        P = dict(prepare=True)
        c, lr, fe = self.compute, self.lr, self.fe
        bx = [self.dense_raw] + self.b_out[:-1]
        tx = [fe.R] + self.t_out[:-1]
        self._fwd_bottom = [ctr.ctr_dense_fwd(x, L.W, L.b, L.relu, c, y, **P)
                            for L, x, y in zip(self.bottom, bx, self.b_out)]
        self._fwd_top = [ctr.ctr_dense_fwd(x, L.W, L.b, L.relu, c, y, **P)
                         for L, x, y in zip(self.top, tx, self.t_out)]
        self._head = ctr.ctr_logistic_ne(self.logits, self.labels, self.prob, self.dlogits,
                                         self.stats, **P)
        t_dy = self.t_dx[1:] + [self.dlogits]
        self._bwd_top = [ctr.ctr_dense_bwd_sgd(x, L.W, L.b, L.relu, y, dy, lr, c, dx,
                                               workspace=self.ws, **P)
                         for L, x, y, dy, dx in zip(self.top, tx, self.t_out, t_dy, self.t_dx)]
        b_dy = self.b_dx[1:] + [fe.dZ[:, 0, :]]
        self._bwd_bottom = [ctr.ctr_dense_bwd_sgd(x, L.W, L.b, L.relu, y, dy, lr, c, dx,
                                                  workspace=self.ws, **P)
                            for L, x, y, dy, dx in zip(self.bottom, bx, self.b_out, b_dy,
                                                       self.b_dx)]

    def forward(self, after_pool=None):
        """Bottom MLP, pooling, interaction, top MLP and head (the head also leaves the
        logits' gradient).  `after_pool` runs right after the pooling call."""
        for call in self._fwd_bottom:
            call()
        fe = self.fe
        if fe.fused_fwd:
            fe._embbag_interaction_fwd()
            if after_pool:
                after_pool()
        else:
            fe._embbag_fwd()
            if after_pool:
                after_pool()
            fe._interaction_fwd()
        for call in self._fwd_top:
            call()
        self._head()

    def backward(self):
        """Everything after the head; the batch's unique must already be enqueued (step()
        does that).  With overlap, the bottom MLP's backward (which reads dZ[:, 0, :] only)
        runs on the side stream beside the embedding backward (dZ[:, 1:, :]) and joins
        before the step ends."""
        for call in reversed(self._bwd_top):
            call()
        fe = self.fe
        fe._interaction_bwd()
        if self.overlap:
            main = torch.cuda.current_stream(self.device)
            main.wait_stream(self.side)                  # the unique is done
            self.side.wait_stream(main)                  # dZ is written
            with torch.cuda.stream(self.side):
                for call in reversed(self._bwd_bottom):
                    call()
            fe._embbag_bwd_sgd()
            main.wait_stream(self.side)
        else:
            fe._embbag_bwd_sgd()
            for call in reversed(self._bwd_bottom):
                call()

    def step(self):
        """One training step: forward, head, backward with every SGD update."""
        fe = self.fe
        if not self.overlap:
            fe.unique()
            self.forward()
            self.backward()
            return

        def fork_unique():
            # the unique of this batch on the side stream, after everything enqueued so far
            # (so after the previous step's backward, which read the unique outputs)
            main = torch.cuda.current_stream(self.device)
            self.side.wait_stream(main)
            with torch.cuda.stream(self.side):
                fe.unique()

        if self.unique_at == "start":
            fork_unique()
            self.forward()
        else:
            self.forward(after_pool=fork_unique)
        self.backward()

    def mlp_only(self):
        """The dense part alone (both MLPs forward and backward and the head), for timing
        the matrix-core work by itself."""
        for call in self._fwd_bottom:
            call()
        for call in self._fwd_top:
            call()
        self._head()
        for call in reversed(self._bwd_top):
            call()
        for call in reversed(self._bwd_bottom):
            call()

    def capture(self, steps: int = 1, fn=None):
        """Record `steps` repetitions of step() (or `fn`) into one HIP graph."""
        fn = fn or self.step
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                fn()
        return g

    def mlp_flops(self) -> float:
        """Multiply-add work of the MLPs per step, counted as 2 flops each: forward X W^T,
        and backward dA W (all but the first bottom layer) and dA^T X."""
        B = self.w.batch
        f = 0.0
        for i, L in enumerate(self.bottom + self.top):
            mats = 3 if i > 0 else 2
            f += 2.0 * B * L.K * L.N * mats
        return f

    def parameters(self) -> List[torch.Tensor]:
        return [t for L in self.bottom + self.top for t in (L.W, L.b)]
