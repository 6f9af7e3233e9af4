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


SR_SEED = 0x5EED_0000_5EED_0005   # base seed of the stochastic-rounding bits


class FrontEnd:
    """Device state for one workload: the tables, the batch and every buffer of the path."""

    def __init__(self, w: Workload, device="cuda", table: Optional[torch.Tensor] = None,
                 fused: bool = True, keep_grads: bool = False, pipelined: bool = False,
                 rounding: str = "nearest", sr_seed: int = SR_SEED, pad_r: bool = False,
                 fused_fwd: bool = False, lean_unique: bool = False,
                 src_rows: Optional[bool] = None, z_bf16: bool = False):
        """fused: the backward applies the sparse SGD as each row gradient completes
        (ctr_embbag_bwd_sgd); otherwise ctr_embbag_bwd then ctr_sparse_sgd.  keep_grads: also
        keep the per-row gradients in self.row_grads (always kept when not fused).
        pipelined: the unique outputs are double-buffered so that step_pipelined() can
        deduplicate the next batch's IDs while the current batch trains.
        rounding: "nearest", or "stochastic" (bf16 or fp16 tables): the k-th update of the
        run (the native step k, or the k-th SGD stage run from Python) draws its rounding bits
        with seed ctr_sr_step_seed(sr_seed, k).
        pad_r: R's rows start on 16-byte boundaries (stride rounded up to 4 floats), so that a
        layer reading R loads it with vector loads; R is then a strided view (the native step
        runner, which assumes contiguous R, refuses it).
        fused_fwd: the forward is one call, ctr_embbag_interaction_fwd (pooling into Z and the
        interaction from an on-chip copy of the pooled vectors), instead of ctr_embbag_fwd
        then ctr_dot_interaction_fwd (pooled-interaction workloads only).
        lean_unique: the pooled step's unique (Python-driven and native) produces only what
        its backward reads (distinct rows, their count, sorted_src): no inverse map,
        permutation or segment offsets, and no occurrence payload through the sort.
        src_rows: sorted_src holds 8-byte row entries (CTR_SRC_ROWS) instead of 16-byte
        (u, bag, key) quadruples; only for the fused update without kept gradients, which is
        also the default (None) then.
        z_bf16: Z (the dense and pooled vectors) is held in bf16 (matrix-core workloads with the
        two-call forward): the pooling rounds its fp32 sums once at the store, the interaction
        reads the same operands it would round from fp32, in half the bytes."""
        assert rounding in ("nearest", "stochastic")
        assert rounding == "nearest" or w.dtype in ("bf16", "f16"), \
            "stochastic rounding: bf16 or fp16 tables"
        self.rounding = rounding
        self.lean_unique = lean_unique

        self.sr_seed = sr_seed
        self._sr_k = 0
        self.w = w
        self.pipelined = pipelined
        self.fused = fused
        self.fused_fwd = bool(fused_fwd and w.interaction)
        assert not z_bf16 or (w.interaction and w.compute == "bf16" and not self.fused_fwd), \
            "a bf16 Z: matrix-core interaction and the two-call forward"
        self.z_bf16 = z_bf16
        self.keep_grads = keep_grads or not fused
        if src_rows is None:
            src_rows = self.fused and not self.keep_grads
        assert not src_rows or (self.fused and not self.keep_grads), \
            "row entries serve the fused update without row gradients"
        self.src_rows = src_rows
        self.device = torch.device(device)
        self.compute = ctr.CTR_BF16 if w.compute == "bf16" else ctr.CTR_F32
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]
        if table is None:
            table = torch.empty((w.total_rows, w.dim), dtype=tdt, device=self.device)
            ctr.ctr_init_tables_hash(table, w.rows, w.table_seed)
        self.table = table
        self.row_base = _dev(w.row_base, self.device)
        self.indices = _dev(w.indices, self.device)
        self.offsets = _dev(w.offsets, self.device)
        self.nnz = w.nnz
        B, T, d = w.batch, w.num_tables, w.dim
        if w.interaction:
            F = w.F
            self.Z = torch.empty((B, F, d), dtype=torch.bfloat16 if z_bf16 else torch.float32,
                                 device=self.device)
            self.Z[:, 0, :].copy_(_dev(w.dense, self.device))        # batch upload
            width = d + w.P
            stride = (width + 3) // 4 * 4 if pad_r else width
            self.R = torch.empty((B, stride), dtype=torch.float32,
                                 device=self.device)[:, :width]
            self.pad_r = pad_r and stride != width
            self.dR = _dev(w.grad_out, self.device)
            # a bf16 interaction keeps its gradient in bf16 (the backward re-reads it per
            # occurrence and sums in fp32)
            self.dZ = torch.empty(self.Z.shape, device=self.device,
                                  dtype=torch.bfloat16 if self.compute == ctr.CTR_BF16
                                  else torch.float32)
        else:
            n = w.nnz
            self.E = torch.empty((max(n, 1), d), dtype=torch.float32, device=self.device)
            self.out = torch.empty((max(n, 1), d), dtype=torch.float32, device=self.device)
            self.dout = _dev(w.grad_out.reshape(n, d), self.device)
        self.row_grads = (torch.empty((max(self.nnz, 1), d), dtype=torch.float32,
                                      device=self.device) if self.keep_grads else None)
        n = self.nnz
        dv = self.device
        self.ws_unique = torch.empty(max(ctr.unique_workspace_bytes(n), 256), dtype=torch.uint8,
                                     device=dv)
        self.ws_bwd = torch.empty(max(ctr.embbag_bwd_workspace_bytes(n, d), 256),
                                  dtype=torch.uint8, device=dv)
        self.ws_pool = torch.zeros(max(ctr.embbag_fwd_workspace_bytes(max(n, 1), d), 256),
                                   dtype=torch.uint8, device=dv)
        self._sets = [self._unique_buffers(n, dv, 2 if src_rows else 4)
                      for _ in range(3 if pipelined else 1)]
        self._calls = []
        self.side = None
        self._k = 0
        for i in range(len(self._sets)):
            self._use_set(i)
            self._prepare()
            self._calls.append({k: v for k, v in self.__dict__.items() if k.startswith("_c_")})
        self._use_set(0)

    @staticmethod
    def _unique_buffers(n, dv, src_words):
        return dict(uniq=torch.empty(max(n, 1), dtype=torch.int64, device=dv),
                    inverse=torch.empty(max(n, 1), dtype=torch.int32, device=dv),
                    num_unique=torch.zeros(1, dtype=torch.int32, device=dv),
                    perm=torch.empty(max(n, 1), dtype=torch.int32, device=dv),
                    seg=torch.empty(n + 1, dtype=torch.int32, device=dv),
                    sorted_src=torch.empty((max(n, 1), src_words), dtype=torch.int32,
                                           device=dv))

    def _use_set(self, i):
        """Point the unique outputs, and the prepared calls that use them, at set i."""
        for k, v in self._sets[i].items():
            setattr(self, k, v)
        # lean_unique (pooled step): the unique fills what the backward reads, not the inverse
        # map, the permutation or the segment offsets
        lean = self.lean_unique and self.w.interaction
        self._unique_out = (self.uniq, None if lean else self.inverse, self.num_unique,
                            None if lean else self.perm, None if lean else self.seg)
        if len(self._calls) > i:
            for k, v in self._calls[i].items():
                setattr(self, k, v)

    # ------------------------------------------------------------------ steps of the path
    def _prepare(self):
        """Marshal every call of the step once (buffers never move)."""
        w = self.w
        d = w.dim
        P = dict(prepare=True)
        if w.interaction:
            F = w.F
            self._c_unique = ctr.ctr_unique_ids(
                self.indices, offsets=self.offsets, batch=w.batch, num_tables=w.num_tables,
                row_base=self.row_base, total_rows=w.total_rows, max_table_rows=max(w.rows),
                workspace=self.ws_unique, out=self._unique_out, sorted_src=self.sorted_src, **P)
            self._c_embbag_fwd = ctr.ctr_embbag_fwd(
                self.table, self.indices, self.offsets, w.batch, w.num_tables, self.Z[:, 1:, :],
                F * d, d, row_base=self.row_base, workspace=self.ws_pool, **P)
            self._c_interaction_fwd = ctr.ctr_dot_interaction_fwd(self.Z, self.compute, self.R, **P)
            # the fused forward writes an fp32 Z
            self._c_embbag_interaction_fwd = None if self.z_bf16 else ctr.ctr_embbag_interaction_fwd(
                self.table, self.indices, self.offsets, self.Z, self.compute, self.R,
                row_base=self.row_base, **P)
            self._c_interaction_bwd = ctr.ctr_dot_interaction_bwd(self.Z, self.dR, self.compute,
                                                                  self.dZ, **P)
            if not self.fused:
                self._c_embbag_bwd = ctr.ctr_embbag_bwd(
                    self.dZ[:, 1:, :], F * d, d, self.offsets, w.batch, w.num_tables, d, None,
                    None, self.num_unique, self.row_grads, workspace=self.ws_bwd,
                    sorted_src=self.sorted_src, nnz=self.nnz, **P)
        else:
            self._c_unique = ctr.ctr_unique_ids(
                self.indices, key_modulus=w.key_modulus, workspace=self.ws_unique,
                out=self._unique_out, sorted_src=self.sorted_src, **P)
            self._c_gather_rows = ctr.ctr_gather_rows(self.table, self.uniq, self.num_unique,
                                                      self.nnz, out=self.E, **P)
            self._c_embbag_fwd = ctr.ctr_embbag_fwd(self.E, self.inverse, self.offsets, self.nnz,
                                                    1, self.out, d, 0, workspace=self.ws_pool,
                                                    **P)
            if not self.fused:
                self._c_embbag_bwd = ctr.ctr_embbag_bwd(
                    self.dout, d, 0, self.offsets, self.nnz, 1, d, None, None,
                    self.num_unique, self.row_grads, workspace=self.ws_bwd,
                    sorted_src=self.sorted_src, nnz=self.nnz, **P)
        if self.fused:
            if w.interaction:
                F = w.F
                grad, sb, st, B, T = self.dZ[:, 1:, :], F * d, d, w.batch, w.num_tables
            else:
                grad, sb, st, B, T = self.dout, d, 0, self.nnz, 1
            self._c_embbag_bwd_sgd = ctr.ctr_embbag_bwd_sgd(
                grad, sb, st, self.offsets, B, T, self.nnz, self.sorted_src, self.num_unique,
                self.table, self.uniq, w.lr, row_grads=self.row_grads, workspace=self.ws_bwd,
                **P)
        else:
            self._c_sparse_sgd = ctr.ctr_sparse_sgd(self.table, self.uniq, self.num_unique,
                                                    self.nnz, self.row_grads, w.lr, **P)

    def unique(self):
        self._c_unique()

    def _embbag_fwd(self):
        self._c_embbag_fwd()

    def _gather_rows(self):
        self._c_gather_rows()

    def _interaction_fwd(self):
        self._c_interaction_fwd()

    def _embbag_interaction_fwd(self):
        self._c_embbag_interaction_fwd()

    def _interaction_bwd(self):
        self._c_interaction_bwd()

    def _embbag_bwd(self):
        self._c_embbag_bwd()

    def _sparse_sgd(self):
        if self.rounding == "stochastic":
            ctr.ctr_sparse_sgd(self.table, self.uniq, self.num_unique, self.nnz,
                               self.row_grads, self.w.lr, ctr.CTR_ROUND_STOCHASTIC,
                               self._sr_seed_next())
            return
        self._c_sparse_sgd()

    def _sr_seed_next(self) -> int:
        seed = ctr.ctr_sr_step_seed(self.sr_seed, self._sr_k)
        self._sr_k += 1
        return seed

    def _embbag_bwd_sgd(self):
        if self.rounding == "stochastic":      # a fresh seed per update: marshalled per call
            w = self.w
            d = w.dim
            if w.interaction:
                grad, sb, st, B, T = self.dZ[:, 1:, :], w.F * d, d, w.batch, w.num_tables
            else:
                grad, sb, st, B, T = self.dout, d, 0, self.nnz, 1
            ctr.ctr_embbag_bwd_sgd(grad, sb, st, self.offsets, B, T, self.nnz,
                                   self.sorted_src, self.num_unique, self.table, self.uniq,
                                   w.lr, row_grads=self.row_grads, workspace=self.ws_bwd,
                                   rounding=ctr.CTR_ROUND_STOCHASTIC,
                                   seed=self._sr_seed_next())
            return
        self._c_embbag_bwd_sgd()

    def stages(self):
        """The step's calls in dependency order, as (name, fn)."""
        tail = ([("embbag_bwd_sgd", self._embbag_bwd_sgd)] if self.fused else
                [("embbag_bwd", self._embbag_bwd), ("sparse_sgd", self._sparse_sgd)])
        if self.w.interaction:
            fwd = ([("embbag_interaction_fwd", self._embbag_interaction_fwd)] if self.fused_fwd
                   else [("embbag_fwd", self._embbag_fwd),
                         ("interaction_fwd", self._interaction_fwd)])
            return fwd + [("interaction_bwd", self._interaction_bwd),
                          ("unique", self.unique)] + tail
        return [("unique", self.unique), ("gather_rows", self._gather_rows),
                ("embbag_fwd", self._embbag_fwd)] + tail

    def forward(self):
        if self.fused_fwd:
            self._embbag_interaction_fwd()
        elif self.w.interaction:
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
        if self.fused:
            self._embbag_bwd_sgd()
        else:
            self._embbag_bwd()
            self._sparse_sgd()

    def run(self, names, mark=None):
        """Run the named stages in step order.  With tables and a dense vector the batch's
        unique runs on a second stream (default priority), forked when the segment starts
        and joined before its first consumer (or at the end of the segment), so it overlaps
        the forward and the interaction gradient.  ``mark(name, fn)`` may wrap a stage."""
        go = mark if mark is not None else (lambda name, fn: fn())
        fns = dict(self.stages())
        order = [n for n, _ in self.stages() if n in names]
        if not self.w.interaction or "unique" not in order:
            for n in order:
                go(n, fns[n])
            return
        main = torch.cuda.current_stream(self.device)
        if self.side is None:
            self.side = torch.cuda.Stream(device=self.device)
        self.side.wait_stream(main)
        with torch.cuda.stream(self.side):
            go("unique", self.unique)
        pending = True
        for n in order:
            if n == "unique":
                continue
            if pending and n in ("embbag_bwd", "sparse_sgd", "embbag_bwd_sgd"):
                main.wait_stream(self.side)
                pending = False
            go(n, fns[n])
        if pending:
            main.wait_stream(self.side)

    def step(self, mark=None):
        """One training step (all stages)."""
        self.run([n for n, _ in self.stages()], mark)

    def split(self, at: str):
        """Stage names before `at`, and after it, such that the unique lands in a segment
        that precedes its consumers.  Used to time one kernel between captured segments."""
        names = [n for n, _ in self.stages()]
        main = [n for n in names if n != "unique"] if self.w.interaction else names
        if at == "unique":
            i = names.index("unique")
            return names[:i], names[i + 1:]
        i = main.index(at)
        pre, post = main[:i], main[i + 1:]
        if self.w.interaction:            # the unique goes with the earliest segment
            if pre:
                pre = pre + ["unique"]
            else:
                post = post + ["unique"]
        return pre, post

    # ------------------------------------------------------------ pipelined schedule
    def pipeline_start(self):
        """Deduplicate the first batch; then call step_pipelined() once per batch."""
        assert self.pipelined, "FrontEnd(pipelined=True) required"
        if self.side is None:
            self.side = torch.cuda.Stream(device=self.device)
        self._k = 0
        self._use_set(0)
        self.unique()

    def capture_pipelined_parts(self, fork_after: str):
        """Graphs for a pipelined step, one of each per buffer set: the unique (replayed on the
        side stream) and the main-stream stages after `fork_after` (replayed on the current
        stream).  The stages up to `fork_after` stay eager, so HIP events can bracket them;
        step_pipelined() then forks the next batch's unique right after them."""
        if self.side is None:
            self.side = torch.cuda.Stream(device=self.device)
        names = [n for n, _ in self.stages() if n != "unique"]
        i = names.index(fork_after) + 1
        self._fork_after = fork_after
        self._eager_names, rest = names[:i], names[i:]
        self._g_unique, self._g_rest = [], []
        for cur in range(len(self._sets)):
            self._use_set(cur)
            self._g_unique.append(self.capture(["unique"]))
            self._g_rest.append(self.capture(rest) if rest else None)
        self._use_set(0)

    def step_pipelined(self, mark=None, k: Optional[int] = None,
                       fork_after: Optional[str] = None):
        """Step k of a stream of batches: batch k trains on the unique outputs computed during
        step k-1 (set k % 2) while batch k+1's unique fills the other set on the side stream,
        forked when the step starts (or right after stage `fork_after`) and joined when it
        ends.  Every call of the path runs exactly once per step.  (The synthetic stream
        repeats one batch, so batch k+1 holds the same IDs.)  After capture_pipelined_parts()
        the unique and the stages after the fork replay from the graphs of their sets."""
        go = mark if mark is not None else (lambda name, fn: fn())
        if k is None:
            k = self._k
        cur, nxt = k & 1, (k + 1) & 1
        main = torch.cuda.current_stream(self.device)
        graphs = getattr(self, "_g_unique", None)
        if graphs:
            fork_after = self._fork_after
        self._k = k + 1

        def fork():
            self.side.wait_stream(main)
            with torch.cuda.stream(self.side):
                if graphs:
                    graphs[nxt].replay()
                else:
                    self._use_set(nxt)
                    self.unique()
            self._use_set(cur)

        self._use_set(cur)
        if fork_after is None:
            fork()
        for n, fn in self.stages():
            if n == "unique" or (graphs and n not in self._eager_names):
                continue
            go(n, fn)
            if n == fork_after:
                fork()
        if graphs and self._g_rest[cur] is not None:
            self._g_rest[cur].replay()
        main.wait_stream(self.side)

    def capture_pipelined(self, steps: int = 2):
        """Record `steps` (even) consecutive pipelined steps, starting with an even step, into
        one HIP graph; each replay continues the stream of batches."""
        assert steps % 2 == 0
        if self.side is None:
            self.side = torch.cuda.Stream(device=self.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(steps):
                self.step_pipelined(k=k)
        self._k = 0
        return g

    # ------------------------------------------------------------ native step
    def native(self) -> ctr.CtrStep:
        """The step's buffers as a ctr_step_t for ctr_step_run (built once)."""
        if getattr(self, "_native", None) is not None:
            return self._native
        assert not getattr(self, "pad_r", False), "the native step runner needs contiguous R"
        assert not self.fused_fwd, "the native step runner makes the two forward calls"
        w = self.w
        d = ctr.CtrStep()
        P = lambda t: None if t is None else t.data_ptr()
        d.kind = ctr.CTR_STEP_POOLED_INTERACTION if w.interaction else ctr.CTR_STEP_BATCH_MATRIX
        d.index_type = ctr.CTR_I64 if self.indices.dtype == torch.int64 else ctr.CTR_I32
        d.indices, d.nnz, d.offsets = P(self.indices), self.nnz, P(self.offsets)
        d.batch, d.num_tables, d.dim = w.batch, w.num_tables, w.dim
        d.row_base, d.key_modulus = P(self.row_base), w.key_modulus
        d.max_table_rows = max(w.rows) if w.interaction else 0
        d.table, d.dtype, d.compute = P(self.table), ctr._dtype_code(self.table), self.compute
        d.total_rows, d.lr = w.total_rows, w.lr
        d.rounding = (ctr.CTR_ROUND_STOCHASTIC if self.rounding == "stochastic"
                      else ctr.CTR_ROUND_NEAREST)
        d.sr_seed = self.sr_seed
        if w.interaction:
            d.Z, d.R, d.dR, d.dZ = P(self.Z), P(self.R), P(self.dR), P(self.dZ)
            d.grad_dtype = ctr._dtype_code(self.dZ)
            d.z_dtype = ctr._dtype_code(self.Z)
        else:
            d.E, d.out, d.dout = P(self.E), P(self.out), P(self.dout)
        d.row_grads = P(self.row_grads)
        d.ws_unique, d.ws_unique_bytes = P(self.ws_unique), self.ws_unique.numel()
        if self.pipelined:            # the two-deep schedule runs two uniques at once
            self.ws_unique2 = torch.empty_like(self.ws_unique)
            d.ws_unique2, d.ws_unique2_bytes = P(self.ws_unique2), self.ws_unique2.numel()
        d.ws_bwd, d.ws_bwd_bytes = P(self.ws_bwd), self.ws_bwd.numel()
        d.ws_pool, d.ws_pool_bytes = P(self.ws_pool), self.ws_pool.numel()
        # The pooled step's unique produces what its backward reads: the distinct rows, their
        # count and sorted_src.  The inverse map, the permutation and the segment offsets are
        # for the batch-matrix step (which pools through the inverse) and for callers that ask.
        lean = w.interaction and self.lean_unique
        for i in range(3):
            b = self._sets[min(i, len(self._sets) - 1)]
            d.uniq[i], d.num_unique[i] = P(b["uniq"]), P(b["num_unique"])
            d.inverse[i] = None if lean else P(b["inverse"])
            d.perm[i] = None if lean else P(b["perm"])
            d.seg_offsets[i] = None if lean else P(b["seg"])
            d.sorted_src[i] = P(b["sorted_src"])
        d.src_layout = ctr.CTR_SRC_ROWS if self.src_rows else ctr.CTR_SRC_FULL
        self._native = d
        self._ev_fork, self._ev_join = torch.cuda.Event(), torch.cuda.Event()
        self._ev_fork.record()          # torch creates the HIP event on its first record
        self._ev_join.record()
        if self.side is None:
            self.side = torch.cuda.Stream(device=self.device)
        # the two-deep schedule: a second side stream and six events carried between steps
        self.side2 = torch.cuda.Stream(device=self.device)
        self._ev_deep = [torch.cuda.Event() for _ in range(6)]
        for e in self._ev_deep:
            e.record()
        return d

    def native_start(self, deep: bool = False):
        """Prime the native pipelined schedules: the first batch's unique into set 0, and for
        the two-deep schedule ("overlap2") the second batch's into set 1, on the current
        stream."""
        d = self.native()
        ctr.ctr_step_unique(d, 0)
        if deep:
            ctr.ctr_step_unique(d, 1)
        self._k = 0

    SCHEDULES = {"serial": ctr.CTR_SCHEDULE_SERIAL,
                 "after-pooling": ctr.CTR_SCHEDULE_PIPELINED,
                 "early": ctr.CTR_SCHEDULE_PIPELINED_EARLY,
                 "overlap": ctr.CTR_SCHEDULE_PIPELINED_OVERLAP,
                 "overlap2": None}                 # ctr_step_run_deep

    def _run_native(self, k: int, schedule: str, stream, mark_begin=None, mark_end=None,
                    side=None):
        d = self.native()
        if schedule == "overlap2":
            ctr.ctr_step_run_deep(d, k, stream, [self.side, self.side2], self._ev_deep,
                                  mark_begin, mark_end)
        else:
            ctr.ctr_step_run(d, k, self.SCHEDULES[schedule], stream,
                             side if side is not None else self.side, self._ev_fork,
                             self._ev_join, mark_begin, mark_end)

    def _set_of(self, k: int, schedule: str) -> int:
        if schedule == "serial":
            return 0
        return k % 3 if schedule == "overlap2" else k & 1

    def step_native(self, schedule: str = "serial", mark_begin=None, mark_end=None):
        """One whole step in one native call (ctr_step_run, or ctr_step_run_deep for
        "overlap2") under `schedule` (a key of SCHEDULES; the pipelined ones need
        FrontEnd(pipelined=True) and native_start() before the first step, native_start(
        deep=True) for "overlap2"); mark_begin/mark_end (optional torch.cuda.Event) bracket
        the pooling kernel.  After it, the unique outputs of the step's batch are the
        attributes.  With the overlapped schedules the next batches' uniques may still be
        running on the side streams: native_join() (or a device synchronize) before reading
        them."""
        pipelined = schedule != "serial"
        assert self.pipelined or not pipelined, "the pipelined schedules need the buffer sets"
        k = self._k
        self._run_native(k, schedule, torch.cuda.current_stream(self.device), mark_begin,
                         mark_end)
        self._use_set(self._set_of(k, schedule))
        self._k = k + 1

    def native_join(self):
        """Make the current stream wait for the side streams (the overlapped uniques)."""
        cur = torch.cuda.current_stream(self.device)
        cur.wait_stream(self.side)
        if getattr(self, "side2", None) is not None:
            cur.wait_stream(self.side2)

    def capture_native(self, steps: int, schedule: str = "serial", marks=None, side=None):
        """Record `steps` consecutive native steps (k = 0 .. steps-1; an even count for the
        one-deep pipelined schedules, whose set 0 must be primed before each replay; sets 0
        and 1 for "overlap2") into one HIP graph, ending with a join of the side streams.
        marks: optional list of 2*steps timing events around each step's pooling kernel, left
        timed by every replay."""
        assert schedule in self.SCHEDULES
        assert schedule == "serial" or (self.pipelined and (schedule == "overlap2" or
                                                            steps % 2 == 0))
        self.native()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream(self.device)
            for i in range(steps):
                m0 = marks[2 * i] if marks else None
                m1 = marks[2 * i + 1] if marks else None
                self._run_native(i, schedule, cap, m0, m1, side)
            cap.wait_stream(side if side is not None else self.side)
            if schedule == "overlap2":
                cap.wait_stream(self.side2)
        self._use_set(0)
        return g

    def capture(self, names=None, steps: int = 1):
        """Record `steps` repetitions of the named stages (default: the whole step) into one
        HIP graph; replay with .replay().  The step allocates nothing, so the graph holds
        only the library's kernel launches and the stream fork/join."""
        if names is None:
            names = [n for n, _ in self.stages()]
        if self.w.interaction and self.side is None:
            self.side = torch.cuda.Stream(device=self.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                self.run(names)
        return g
