#!/usr/bin/env python3
"""Benchmark of the sparse front end of a CTR ranking model on one MI355X.

A step is one pass of the whole path over one batch of seeded synthetic input, with inputs
already resident in HBM:
  DLRM-shaped workloads:  embbag_fwd -> interaction_fwd -> interaction_bwd -> unique ->
                          embbag_bwd -> sparse_sgd
  TensorNet workload:     unique -> gather_rows -> embbag_fwd (per-slot) -> embbag_bwd ->
                          sparse_sgd
Prints one JSON line: rows gathered per second over whole steps (value), HBM GB/s of the
algorithmic bytes, interaction samples/s, the roofline of the dominant kernel (timed with
HIP events on its stream inside the timed region) and the CPU oracle timed on a bounded
sample of the same workload.

Schedule (default "pipelined"): training consumes a stream of batches, and the ID dedup of
batch k+1 needs only that batch's IDs, so it runs on a second stream during step k into a
second set of output buffers; each timed step still launches every call of the path once.
--pipeline overlap (default) waits for a batch's dedup only before that batch's backward, and
lets the dedup of batch k+2 start once the backward of batch k has released its buffers, so
consecutive steps overlap; early / after-pooling fork the dedup when the step starts / after
the pooling kernel and join it at the step's end.  "serial" dedups each
batch inside its own step; --compare-serial adds that schedule's ms per step to a pipelined
run.

Launch (default "graph"): ctr_step_run enqueues a whole step from C++ (every kernel, the
fork/join of the side stream, and HIP events around the pooling kernel on its stream); the K
timed steps are captured once as one HIP graph, the timing events as event-record nodes, and
the graph is replayed, so the host's launch cost (about 2.5 us per kernel and 10 us per
cross-stream wait on this stack) stays off the steps.  "native" calls ctr_step_run once per
step; "python" makes one binding call per stage (the pipelined schedule then replays the next
batch's unique and the stages after the pooling kernel from captured graphs).

    python bench.py [--config large|small|tiny|criteo|tensornet|dictionary] [--steps K]
                    [--warmup W]
                    [--schedule pipelined|serial] [--compare-serial]
                    [--launch native|python|graph]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published
WORKLOAD_NAMES = {
    "tiny": "Tiny: 4 fp32 tables x 1000 x d16, B=128, one-hot, F=5",
    "small": "Small DLRM-shaped: 8 fp32 tables x 1M x d64, B=2048, Poisson(20) bags, Zipf(1.05), F=9",
    "criteo": "Criteo-shaped: 26 bf16 tables (1e3..1e7 rows) x d128, B=8192, F=27",
    "tensornet": "TensorNet batch-unique: 65536 x 100 IDs, Zipf(1.2) over 1e11, mod 2e7, fp32 d32",
    "large": "Large: 64 bf16 tables x 4M x d128, B=32768, Poisson(32) bags, Zipf(1.1), F=65",
    "dictionary": "Inference lookup: 65536 x 100 raw IDs, Zipf(1.2) over 1e11, in an exported "
                  "dictionary of the 2e7 most popular IDs (fp32 d32), the 2e6 hottest cached in HBM",
}


def grad_elem_bytes(w):
    """Bytes per gradient value the backward reads: the matrix-core interaction stores dZ in
    bf16 (the step's gradient dtype for bf16 compute), everything else is fp32."""
    return 2 if (w.interaction and w.compute == "bf16") else 4


def compulsory_bytes(w, U, stage, z_bytes=4):
    """The stage's bytes with each distinct row read once: the pooled gather reads U rows
    instead of nnz; the fused backward reads each bag's gradient row once (T*B rows, or one
    per occurrence without bags) instead of once per occurrence."""
    n, d = w.nnz, w.dim
    rb = d * (2 if w.dtype == "bf16" else 4)
    if stage == "embbag_bwd_sgd":
        rows = w.num_tables * w.batch if w.interaction else n
        return rows * d * grad_elem_bytes(w) + 8 * n + 2 * U * rb
    assert stage == "embbag_fwd"
    if w.interaction:
        nb = w.num_tables * w.batch
        return U * rb + 8 * n + 8 * (nb + 1) + z_bytes * nb * d
    return U * 4 * d + 4 * n + 8 * (n + 1) + 4 * n * d


def stage_bytes(w, U, src_bytes=16, z_bytes=4):
    """Algorithmic bytes moved by each stage (what the method must read and write).  The
    fused backward + SGD counts every occurrence's gradient row (at the gradient's element
    size), the occurrence's 8-byte index, and the read and write of each updated row.
    src_bytes: bytes per sorted position of the unique's output for the backward (16 for
    (u, bag, key) quadruples, 8 for row entries).  z_bytes: bytes per value of Z (4, or 2 for
    a bf16 Z)."""
    n = w.nnz
    d = w.dim
    rb = d * (2 if w.dtype == "bf16" else 4)
    sg = grad_elem_bytes(w)
    if w.interaction:
        B, T, F, P = w.batch, w.num_tables, w.F, w.P
        nb = T * B
        return {
            "embbag_fwd": n * rb + 8 * n + 8 * (nb + 1) + z_bytes * nb * d,
            "interaction_fwd": z_bytes * B * F * d + 4 * B * (d + P),
            # dR and Z read, dZ written at its stored width (bf16 for a bf16 backward)
            "interaction_bwd": 4 * B * (d + P) + (z_bytes + sg) * B * F * d,
            # the pooled step's unique: ids and offsets in; the distinct rows and sorted_src
            # (the backward's input, src_bytes per position) out
            "unique": 8 * n + 8 * (nb + 1) + src_bytes * n + 8 * U,
            "embbag_bwd": sg * n * d + 8 * n + 4 * U * d,
            "sparse_sgd": 2 * U * rb + 4 * U * d + 8 * U,
            "embbag_bwd_sgd": sg * n * d + 8 * n + 2 * U * rb,
        }
    return {
        "unique": 8 * n + 4 * n + 4 * n + 12 * U + 4 * U,
        "gather_rows": U * rb + 8 * U + 4 * U * d,
        "embbag_fwd": n * 4 * d + 4 * n + 8 * (n + 1) + 4 * n * d,
        "embbag_bwd": 4 * n * d + 8 * n + 4 * U * d,
        "sparse_sgd": 2 * U * rb + 4 * U * d + 8 * U,
        "embbag_bwd_sgd": sg * n * d + 8 * n + 2 * U * rb,
    }


KERNEL_NAMES = {
    "embbag_fwd": "embbag_fwd_balanced_kernel (pooled gather)",
    "embbag_bwd_sgd": "segreduce_kernel, level 0 (fused backward + sparse SGD)",
}

# Stages that are one kernel launch each (a roofline needs one kernel's duration), with the
# kernel's name prefix and source file.
SINGLE_KERNEL = {
    "embbag_fwd": ("embbag_fwd_", "embbag.hip"),
    # the reduce-by-key level over every sorted position (its carry levels are short)
    "embbag_bwd_sgd": ("segreduce_kernel<true", "segreduce.hip"),
    "interaction_fwd": ("interaction_fwd_", "interaction.hip"),
    "interaction_bwd": ("interaction_bwd_", "interaction.hip"),
    "sparse_sgd": ("sparse_sgd_kernel", "embbag.hip"),
    "gather_rows": ("gather_rows_kernel", "embbag.hip"),
}


class TimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence: HIP documents the flag for
    events that only measure time.  Recording skips the system-scope release, which is a
    cache writeback and invalidation, so the bracket around one kernel is closer to the
    kernel itself.  On the Small workload's pooling kernel this reads 17.0-17.4 us, against
    18.7-19.8 us for a default event, with rocprofv3 at 14.1-15.1 us.  It takes the HIP
    runtime already loaded in the process (the one torch and libctr share), and exposes
    .cuda_event like torch.cuda.Event so that ctr_step_run takes it as a mark."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            path = [ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln][0]
            TimingEvent._hip = ctypes.CDLL(path)
        h = ctypes.c_void_p()
        st = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(h),
                                                      ctypes.c_uint(self.DISABLE_SYSTEM_FENCE))
        if st != 0:
            raise RuntimeError("hipEventCreateWithFlags failed (%d)" % st)
        self.cuda_event = h.value

    def record(self, stream=None):
        import ctypes
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        st = TimingEvent._hip.hipEventRecord(ctypes.c_void_p(self.cuda_event),
                                             ctypes.c_void_p(s.cuda_stream))
        if st != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % st)

    def elapsed_time(self, end) -> float:
        import ctypes
        ms = ctypes.c_float()
        st = TimingEvent._hip.hipEventElapsedTime(ctypes.byref(ms),
                                                  ctypes.c_void_p(self.cuda_event),
                                                  ctypes.c_void_p(end.cuda_event))
        if st != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % st)
        return ms.value


def cpu_baseline_variants(fe, w, seconds: float):
    """The oracle's interaction variants (self-dot pairs, the Gram matrix and the FM sum,
    forward and backward) on the first samples of the workload's Z, repeated until `seconds`
    in total; samples per second for each call."""
    import numpy as np
    from oracle import oracle as orc

    B, F, d = w.batch, w.F, w.dim
    P = F * (F + 1) // 2
    rng = np.random.default_rng(9)
    Zs = fe.Z[:min(B, 4096)].double().cpu().numpy()
    dR = rng.standard_normal((Zs.shape[0], d + P))
    dRg = rng.standard_normal((Zs.shape[0], d + F * F))
    dout = rng.standard_normal(Zs.shape[0])
    calls = {"interaction_self_fwd": lambda z, r, o: orc.interaction_self_fwd(z),
             "interaction_self_bwd": lambda z, r, o: orc.interaction_self_bwd(z, r),
             "interaction_gram_fwd": lambda z, r, o: orc.interaction_gram_fwd(z),
             "interaction_gram_bwd": lambda z, r, o: orc.interaction_gram_bwd(
                 z, dRg[:z.shape[0]]),
             "fm_fwd": lambda z, r, o: orc.fm_fwd(z),
             "fm_bwd": lambda z, r, o: orc.fm_bwd(z, o)}
    res = {}
    for name, fn in calls.items():
        t0 = time.perf_counter()                  # size the sample from a 64-sample call
        fn(Zs[:64], dR[:64], dout[:64])
        t1 = time.perf_counter() - t0
        b = int(min(Zs.shape[0], max(64, 64 * seconds / 4 / max(t1, 1e-6))))
        reps = 0
        t0 = time.perf_counter()
        while True:
            fn(Zs[:b], dR[:b], dout[:b])
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds / 4 or reps >= 100:
                break
        res[name] = {"value": reps * b / el, "unit": "samples/s", "cores": orc.get_threads(),
                     "kind": "oracle", "sample": "%d call(s) on the first %d samples" % (reps, b)}
    return res


def time_variants(fe, w, K: int):
    """The interaction variants on the workload's Z (after the timed steps), each call alone
    bracketed by HIP events: the pair set with self-dots, forward and backward (P = F(F+1)/2),
    the whole Gram matrix (P = F^2), and the FM sum by the squared-norm identity; and the fused
    forward (pooling and the interaction in one call) beside the two calls it replaces, timed
    the same way.  Algorithmic bytes: self and Gram forward 4BFd + 4B(d+P), backward
    4B(d+P) + 8BFd; FM forward 4BFd + 4B, backward 8BFd + 4B; fused forward the pooling's
    bytes plus the dense rows read (4Bd) and R written (4B(d+P)), the separate pair that plus
    Z's re-read (4BFd)."""
    import torch
    from sparse_embedding_lookup_amd import ctr

    B, F, d = w.batch, w.F, w.dim
    P = F * (F + 1) // 2
    gen = torch.Generator(device="cuda").manual_seed(7)
    dR = torch.randn((B, d + P), generator=gen, device="cuda")
    dout = torch.randn((B,), generator=gen, device="cuda")
    R = torch.empty((B, d + P), device="cuda")
    Pg = F * F
    dRg = torch.randn((B, d + Pg), generator=gen, device="cuda")
    Rg = torch.empty((B, d + Pg), device="cuda")
    Zf = fe.Z if fe.Z.dtype == torch.float32 else fe.Z.float()   # the fp32-Z entry points'
    dZ = torch.empty_like(Zf)
    out = torch.empty((B,), device="cuda")
    calls = {
        "interaction_self_fwd": (ctr.ctr_dot_interaction_self_fwd(Zf, fe.compute, R, prepare=True),
                                 4 * B * F * d + 4 * B * (d + P)),
        "interaction_self_bwd": (ctr.ctr_dot_interaction_self_bwd(Zf, dR, fe.compute, dZ,
                                                                  prepare=True),
                                 4 * B * (d + P) + 8 * B * F * d),
        "interaction_gram_fwd": (ctr.ctr_dot_interaction_gram_fwd(Zf, fe.compute, Rg,
                                                                  prepare=True),
                                 4 * B * F * d + 4 * B * (d + Pg)),
        "interaction_gram_bwd": (ctr.ctr_dot_interaction_gram_bwd(Zf, dRg, fe.compute, dZ,
                                                                  prepare=True),
                                 4 * B * (d + Pg) + 8 * B * F * d),
        "fm_fwd": (ctr.ctr_fm_interaction_fwd(Zf, out, prepare=True), 4 * B * F * d + 4 * B),
        "fm_bwd": (ctr.ctr_fm_interaction_bwd(Zf, dout, dZ, prepare=True),
                   8 * B * F * d + 4 * B),
    }
    Pd = F * (F - 1) // 2                              # the strict pair set of the step
    pool = stage_bytes(w, 0)["embbag_fwd"]             # (the fused call's Z is fp32)
    fused = pool + 4 * B * d + 4 * B * (d + Pd)
    fused_call = fe._c_embbag_interaction_fwd
    if fused_call is None:                             # a bf16 Z: the fused call on a copy
        fused_call = ctr.ctr_embbag_interaction_fwd(
            fe.table, fe.indices, fe.offsets, Zf, fe.compute,
            torch.empty((B, d + Pd), device="cuda"), row_base=fe.row_base, prepare=True)
    calls["embbag_interaction_fwd"] = (fused_call, fused)

    def separate():
        fe._c_embbag_fwd()
        fe._c_interaction_fwd()
    zb = 2 if fe.z_bf16 else 4
    sep = stage_bytes(w, 0, z_bytes=zb)
    calls["embbag_fwd+interaction_fwd"] = (separate, sep["embbag_fwd"] + sep["interaction_fwd"])
    res = {}
    for name, (call, nbytes) in calls.items():
        for _ in range(3):
            call()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K)]
        for e0, e1 in ev:
            e0.record()
            call()
            e1.record()
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in ev) / K
        gbps = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 5), "bytes": nbytes, "gbps": round(gbps, 1),
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "compute": "bf16" if fe.compute == ctr.CTR_BF16 and "fm" not in name
                     else "f32"}
    return res


MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense matrix-core peaks


def time_dlrm(fe, w, K: int):
    """The whole DLRM training step around the front end (bottom MLP into Z[:, 0, :], top MLP,
    logistic/NE head, backward with SGD of every parameter), sharing the front end's table:
    K steps captured as one HIP graph and replayed; the dense part alone likewise; and each
    layer's forward and backward call alone, priced against the matrix
    cores' dense peak for the compute type (flops: 2 per multiply-add; forward B K N,
    backward dX and dW 2 B K N, B K N for the first bottom layer, which has no dX).  Times
    are K calls replayed from one HIP graph, divided by K."""
    import torch
    from sparse_embedding_lookup_amd import ctr, workloads
    from sparse_embedding_lookup_amd.dlrm import DlrmStep

    inp = workloads.dlrm_inputs(w)
    s = DlrmStep(w, inp, "cuda", table=fe.table)
    kind = "bf16" if s.compute == ctr.CTR_BF16 else "f32"
    peak = MFMA_PEAK_TFLOPS[kind]
    for _ in range(3):
        s.step()
    torch.cuda.synchronize()

    def graph_ms(fn):
        g = s.capture(steps=K, fn=fn)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / K

    step_ms = graph_ms(s.step)
    mlp_ms = graph_ms(s.mlp_only)
    B = w.batch
    layers = []
    calls = ([("bottom%d" % i, L, f, b, i == 0) for i, (L, f, b) in
              enumerate(zip(s.bottom, s._fwd_bottom, s._bwd_bottom))] +
             [("top%d" % i, L, f, b, False) for i, (L, f, b) in
              enumerate(zip(s.top, s._fwd_top, s._bwd_top))])
    for name, L, fwd, bwd, first in calls:
        row = {"K": L.K, "N": L.N}
        for part, call, mats in (("fwd", fwd, 1), ("bwd", bwd, 1 if first else 2)):
            # K back-to-back calls replayed from a graph: launch gaps do not count
            ms = graph_ms(call)
            tf = 2.0 * B * L.K * L.N * mats / (ms * 1e-3) / 1e12
            row[part + "_ms"] = round(ms, 5)
            row[part + "_tflops"] = round(tf, 1)
            row[part + "_frac"] = round(tf / peak, 4)
        layers.append((name, row))
    flops = s.mlp_flops()
    big = max(layers, key=lambda kv: kv[1]["K"] * kv[1]["N"])
    return {
        "forward": ("fused: ctr_embbag_interaction_fwd" if s.fe.fused_fwd else
                    "separate: ctr_embbag_fwd, ctr_dot_interaction_fwd"),
        "mlp": {"bottom": [13, *workloads.DLRM_BOTTOM, w.dim],
                "top": [w.dim + w.P, *workloads.DLRM_TOP, 1], "compute": kind},
        "step_ms": round(step_ms, 5),
        "rows_per_s": w.nnz / (step_ms * 1e-3),
        "samples_per_s": B / (step_ms * 1e-3),
        "mlp_ms": round(mlp_ms, 5),
        "mlp_tflops": round(flops / (mlp_ms * 1e-3) / 1e12, 1),
        "ne": float(s.stats[2].item()),
        "layers": dict(layers),
        "roofline": {"kernel": big[0] + " backward (dX and dW GEMMs)", "bound": "mfma",
                     "achieved": big[1]["bwd_tflops"], "peak": peak, "unit": "TFLOP/s",
                     "frac": big[1]["bwd_frac"]},
    }


def interaction_block(w, stage_ms, byts):
    """The interaction's forward and backward, each alone between HIP events: algorithmic
    bytes and their fraction of 8 TB/s; with matrix-core compute also the MFMA flops the
    kernels issue (32x32x16 bf16 tiles: the forward's lower-triangle tiles, d/16 each; the
    backward's 32-column slabs x 32-row blocks x 16-row k-steps) and their fraction of the
    2.5 PFLOP/s dense bf16 peak."""
    B, F, d = w.batch, w.F, w.dim
    fb, km, ks, nb = (F + 31) // 32, (F + 15) // 16, d // 16, (d + 31) // 32
    tiles = sum(1 for i in range(fb) for j in range(i + 1) if not (j == i and F - 32 * i < 2))
    mfma = {"interaction_fwd": tiles * ks, "interaction_bwd": nb * fb * km}
    out = {}
    for k in ("interaction_fwd", "interaction_bwd"):
        ms = stage_ms[k]
        gbps = byts[k] / (ms * 1e-3) / 1e9
        e = {"ms": round(ms, 5), "bytes": byts[k], "gbps": gbps, "frac": gbps / HBM_PEAK_GBPS}
        if w.compute == "bf16":
            flops = mfma[k] * 32 * 32 * 16 * 2 * B
            e["mfma_flops"] = flops
            e["mfma_tflops"] = flops / (ms * 1e-3) / 1e12
            e["mfma_frac"] = e["mfma_tflops"] / 2500.0
        out[k] = e
    return out


def measured_traffic(config: str, stage: str):
    """Bytes per launch that the stage's kernel moved between L2 and memory, from the
    committed rocprofv3 counter runs (read requests counted by size, 32/64/128 bytes, and
    write requests), or None when there is no such run or the kernel's source changed since
    it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s.json" % config)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        prof = json.load(f)
    prefix, src = SINGLE_KERNEL[stage]
    csrc = os.path.join(ROOT, "sparse_embedding_lookup_amd", "csrc")
    for fname in (src, "ctr_internal.h"):
        with open(os.path.join(csrc, fname), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest()[:16] != prof["source_sha256_16"].get(fname):
                return None
    for name, v in prof["per_launch"].items():
        if prefix in name:
            return v["fetch_bytes"] + v["write_bytes"]
    return None


def cpu_baseline(w, seconds: float, threads: int = 0):
    """The oracle, as it stands, on repeated full batches until `seconds` of CPU time, on
    `threads` OpenMP threads (0: the oracle's default, every host core)."""
    import numpy as np
    from oracle import oracle as orc

    from sparse_embedding_lookup_amd import workloads

    default_threads = orc.get_threads()
    if threads:
        orc.set_threads(threads)
    try:
        return _cpu_baseline(w, seconds, orc, np, workloads)
    finally:
        if threads:
            orc.set_threads(default_threads)


def _cpu_baseline(w, seconds, orc, np, workloads):
    threads = orc.get_threads()
    tab = orc.Table(w.rows, w.dim, w.dtype, w.table_seed)
    if w.total_rows * w.dim * 4 <= (4 << 30):
        tab = orc.Table(w.rows, w.dim, w.dtype, w.table_seed, data=orc.full_table(tab))
        sample_tab = "host copy of the tables"
        budget = 8_000_000
    else:
        sample_tab = "rows regenerated from the counter-based fill"
        budget = 400_000
    if w.nnz > budget:                     # bound the CPU work: first b samples of the batch
        b = max(1, int(w.batch * budget / w.nnz))
        sample_tab += ", first %d of the %d samples" % (b, w.batch)
        w = workloads.slice_batch(w, b)

    def one_step():
        if w.interaction:
            pooled, _ = orc.embbag_fwd(tab, w.indices, w.offsets, w.batch)
            Z = np.empty((w.batch, w.F, w.dim))
            Z[:, 0] = w.dense
            Z[:, 1:] = pooled
            orc.interaction_fwd(Z)
            dZ, _ = orc.interaction_bwd(Z, w.grad_out)
            keys = orc.form_keys(w.indices, w.offsets, w.num_tables, w.batch, w.row_base)
            uniq, inv, _, _ = orc.unique(keys)
            g, gm = orc.embbag_bwd(dZ[:, 1:], w.offsets, w.batch, w.num_tables, inv, uniq.size)
            orc.sparse_sgd(tab, uniq, g, gm, w.lr)
        else:
            keys = orc.form_keys(w.indices, w.offsets, 1, w.nnz, np.array([0, w.rows[0]]),
                                 w.key_modulus)
            uniq, inv, _, _ = orc.unique(keys)
            E = orc.gather_rows(tab, uniq)
            Et = orc.Table([uniq.size], w.dim, "f32", 0, data=E.astype(np.float32))
            orc.embbag_fwd(Et, inv.astype(np.int64), w.offsets, w.nnz)
            g, gm = orc.embbag_bwd(w.grad_out.reshape(w.nnz, 1, w.dim), w.offsets, w.nnz, 1,
                                   inv, uniq.size)
            orc.sparse_sgd(tab, uniq, g, gm, w.lr)

    reps = 0
    t0 = time.perf_counter()
    while True:
        one_step()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    return {"value": reps * w.nnz / el, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": "%d oracle step(s) over the same batch (%d rows each, %s) in %.1f s"
                      % (reps, w.nnz, sample_tab, el),
            "seconds_per_step": el / reps}


def cpu_baseline_mlp(w, seconds: float):
    """The oracle's MLPs and logistic head (forward, backward and every parameter step) on
    the first samples of the batch, repeated until `seconds`; samples per second."""
    import numpy as np
    from oracle import oracle as orc

    from sparse_embedding_lookup_amd import workloads

    inp = workloads.dlrm_inputs(w)
    R_all = np.random.default_rng(5).standard_normal((min(w.batch, 2048), w.dim + w.P))
    bf16 = w.compute == "bf16"
    nb, nt = len(inp.bottom), len(inp.top)

    def one(b):
        X0 = inp.dense_raw[:b].astype(np.float64)
        R = R_all[:b]
        y = inp.labels[:b]
        acts, x = [], X0
        for i, (W, bb) in enumerate(inp.bottom):
            out, _ = orc.dense_fwd(x, W, bb, True, bf16)
            acts.append((x, out))
            x = out
        x = R
        for i, (W, bb) in enumerate(inp.top):
            out, _ = orc.dense_fwd(x, W, bb, i < nt - 1, bf16)
            acts.append((x, out))
            x = out
        _, dy, _, _, _ = orc.logistic_ne(x[:, 0], y)
        dy = dy[:, None]
        for i in reversed(range(nt)):
            x, out = acts[nb + i]
            W, bb = inp.top[i]
            dy = orc.dense_bwd_sgd(x, W, bb, i < nt - 1, out, dy, bf16, w.lr)["dX"]
        dy = dy[:, :w.dim]                     # the dense slot's share of dR (a stand-in)
        for i in reversed(range(nb)):
            x, out = acts[i]
            W, bb = inp.bottom[i]
            dy = orc.dense_bwd_sgd(x, W, bb, True, out, dy, bf16, w.lr, want_dx=i > 0).get("dX")

    t0 = time.perf_counter()                   # size the sample from a 16-sample pass
    one(16)
    b = int(min(R_all.shape[0], max(16, 16 * 0.5 * seconds / (time.perf_counter() - t0))))
    reps = 0
    t0 = time.perf_counter()
    while True:
        one(b)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    return {"value": reps * b / el, "unit": "samples/s (MLPs + head, forward and backward)",
            "cores": orc.get_threads(), "kind": "oracle",
            "sample": "%d oracle pass(es) over the first %d samples in %.1f s" % (reps, b, el)}


def bench_dictionary(args):
    """One step = the inference lookup of one batch: ctr_dict_lookup (raw ID -> value) then
    ctr_dict_embbag_fwd (pooled rows, one ID per (sample, slot) bag).  `value` is measured
    with the whole dictionary table in HBM; the hierarchical variant, with the table in
    pinned host memory behind the HBM cache, is timed after it and reported beside it."""
    import numpy as np
    import torch
    from sparse_embedding_lookup_amd import ctr, workloads

    ctr.load()
    print("[bench] generating the dictionary workload", file=sys.stderr, flush=True)
    w = workloads.dictionary()
    n, d = w.nnz, w.dim
    cap = ctr.dict_capacity(w.entries)
    table = torch.empty((w.entries, d), dtype=torch.float32, device="cuda")
    ctr.ctr_init_tables_hash(table, [w.entries], w.table_seed)
    rows_dev = torch.from_numpy(w.dict_rows[:w.hot].astype(np.int64)).cuda()
    hot_rows = table[rows_dev].contiguous()
    slots, status = ctr.ctr_dict_build(torch.from_numpy(w.dict_keys).cuda(),
                                       torch.from_numpy(w.dict_rows).cuda(),
                                       torch.from_numpy(w.hot_slots).cuda(), cap)
    assert host_list(status) == [0, 0, 0], host_list(status)
    ids = torch.from_numpy(w.indices).cuda()
    offsets = torch.from_numpy(w.offsets).cuda()
    values = torch.empty(n, dtype=torch.int64, device="cuda")
    out = torch.empty((n, d), dtype=torch.float32, device="cuda")
    c_lookup = ctr.ctr_dict_lookup(ids, slots, cap, values, prepare=True)
    c_pool = ctr.ctr_dict_embbag_fwd(values, n, offsets, n, 1, hot_rows, table, out, d, 0,
                                     prepare=True)
    K = args.steps

    def run(pool_call):
        for _ in range(args.warmup):
            c_lookup()
            pool_call()
        e = [(TimingEvent(), TimingEvent(), TimingEvent()) for _ in range(K)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for a, b, c in e:
            a.record()
            c_lookup()
            b.record()
            pool_call()
            c.record()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / K
        lk = sum(a.elapsed_time(b) for a, b, _ in e) / K
        pl = sum(b.elapsed_time(c) for _, b, c in e) / K
        return ms, lk, pl

    ms, lk_ms, pool_ms = run(c_pool)
    vals = values.cpu().numpy()
    hit = float(np.mean(vals >= 0))
    cached = float(np.mean((vals >= 0) & ((vals >> 32) > 0)))
    # the hierarchical variant: the full table in pinned host memory, behind the HBM cache
    host_table = torch.empty(table.shape, dtype=table.dtype, pin_memory=True)
    host_table.copy_(table)
    c_pool_h = ctr.ctr_dict_embbag_fwd(values, n, offsets, n, 1, hot_rows, host_table, out, d,
                                       0, prepare=True)
    ms_h, _, pool_h_ms = run(c_pool_h)

    rb = 4 * d
    pool_bytes = 8 * n + 8 * (n + 1) + n * rb + 4 * n * d
    lookup_bytes = 8 * n + 16 * n + 8 * n            # IDs, one 16-byte slot per probe, values
    achieved = pool_bytes / (pool_ms * 1e-3) / 1e9
    res = {
        "metric": "embedding rows gathered/s + HBM GB/s (fwd+bwd); interaction samples/s",
        "value": n / (ms * 1e-3), "unit": "rows/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded; tables from the counter-based fill)",
        "config": {"workload": WORKLOAD_NAMES["dictionary"], "name": "dictionary",
                   "batch": w.batch, "slots": w.slots, "entries": w.entries, "hot": w.hot,
                   "dim": d, "nnz": n, "hit_rate": hit, "cache_hit_rate": cached},
        "stage_ms": {"dict_lookup": round(lk_ms, 5), "dict_embbag_fwd": round(pool_ms, 5)},
        "host_tier": {"ms_per_step": ms_h, "rows_per_s": n / (ms_h * 1e-3),
                      "pool_ms": round(pool_h_ms, 5),
                      "rows_from_host": float(hit - cached),
                      "note": "the dictionary table in pinned host memory behind the HBM cache "
                              "(host-link inclusive; not the headline value)"},
        "roofline": {"kernel": "dict_embbag_fwd", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None, "bytes_per_launch": pool_bytes,
                     "avg_launch_ms": pool_ms,
                     "lookup_gbps": lookup_bytes / (lk_ms * 1e-3) / 1e9},
    }
    if not args.no_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline_dictionary(w, args.cpu_seconds)
    print(json.dumps(res))


def host_list(t):
    return [int(x) for x in t.cpu().tolist()]


def cpu_baseline_dictionary(w, seconds: float):
    """The oracle's lookup and pooled lookup on the first 200,000 IDs of the batch, repeated
    until `seconds` of CPU time (the table regenerated from the fill definition)."""
    from oracle import oracle as orc

    m = min(200_000, w.nnz)
    ids = w.indices[:m]
    off = w.offsets[:m + 1]
    tab = orc.Table([w.entries], w.dim, "f32", w.table_seed)
    reps = 0
    t0 = time.perf_counter()
    while True:
        vals = orc.dict_lookup(w.dict_keys, w.dict_rows, w.hot_slots, ids)
        orc.dict_pool(tab, vals, off, m, 1)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 100:
            break
    return {"value": reps * m / el, "unit": "rows/s", "cores": orc.get_threads(),
            "kind": "oracle", "sample": "%d oracle pass(es) over the first %d IDs of the batch "
                                        "(dictionary sorted per pass) in %.1f s" % (reps, m, el)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="large", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--ids", default="zipf", choices=["zipf", "uniform"],
                    help="zipf: the workload's power-law IDs; uniform: the same shapes with "
                         "uniform IDs (the control where caches cannot help)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-1thread-seconds", type=float, default=6.0,
                    help="also time the oracle on one thread (Tiny, Small and Criteo only); "
                         "0 skips it")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="per-stage timings with the caches flushed before every stage "
                         "(1 GiB written and read); 0 skips them")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--detail", default="", help="write per-stage detail JSON here")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="run one device copy of MB MiB first (scale for HBM byte counters)")
    ap.add_argument("--launch", default="graph", choices=["graph", "native", "python"],
                    help="graph: the K timed steps, enqueued by ctr_step_run under stream "
                         "capture, replayed as one HIP graph; native: one ctr_step_run call per "
                         "step; python: one binding call per stage (with captured graph parts "
                         "when pipelined)")
    ap.add_argument("--schedule", default="pipelined", choices=["pipelined", "serial"],
                    help="pipelined: batch k+1's ID dedup runs during step k (double-buffered "
                         "outputs); serial: every step dedups its own batch first")
    ap.add_argument("--pipeline", default="overlap",
                    choices=["overlap2", "overlap", "early", "after-pooling"],
                    help="pipelined schedule of the native step: overlap2 (two batches' "
                         "uniques in flight on two side streams, three output sets), overlap "
                         "(each step waits for "
                         "its batch's unique only before its backward; steps overlap), early "
                         "(the next batch's unique forked at the step start, joined at its "
                         "end) or after-pooling (forked after the pooling kernel)")
    ap.add_argument("--rounding", default="nearest", choices=["nearest", "stochastic"],
                    help="bf16 tables: round the sparse update to nearest-even, or "
                         "stochastically (a fresh counter-based seed per step)")
    ap.add_argument("--no-variants", dest="variants", action="store_false",
                    help="skip timing the interaction variants (self-dots, FM sum) on the "
                         "workload's Z")
    ap.add_argument("--no-dlrm", dest="dlrm", action="store_false",
                    help="skip timing the whole DLRM step (bottom and top MLP, logistic/NE "
                         "head) around the front end; it runs after the timed steps")
    ap.add_argument("--compare-serial", action="store_true",
                    help="after a pipelined run, also time K serial steps (ms_per_step_serial)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.config == "dictionary":
        bench_dictionary(args)
        return

    import torch
    from sparse_embedding_lookup_amd import ctr, workloads
    from sparse_embedding_lookup_amd.pipeline import FrontEnd

    ctr.load()
    print("[bench] generating workload %s" % args.config, file=sys.stderr, flush=True)
    w = workloads.make(args.config) if args.ids == "zipf" else workloads.make(args.config,
                                                                              ids=args.ids)
    print("[bench] nnz=%d, building device state" % w.nnz, file=sys.stderr, flush=True)
    graph = args.launch == "graph"
    native = args.launch in ("native", "graph")
    pipelined = args.schedule == "pipelined"
    sched = args.pipeline if pipelined else "serial"
    deep = sched == "overlap2"
    if graph and pipelined and not deep and args.steps % 2:
        args.steps += 1                  # a pipelined graph holds whole pairs of steps
    if args.rounding == "stochastic" and w.dtype != "bf16":
        print("--rounding stochastic needs a bf16-table workload (criteo, large)", file=sys.stderr)
        sys.exit(2)
    # the pooled step's unique fills what its backward reads (no inverse map: nothing in the
    # pooled step reads it); the batch-matrix step pools through the inverse map
    # matrix-core workloads hold Z in bf16: the operands the interaction takes, in half the bytes
    fe = FrontEnd(w, "cuda", pipelined=pipelined, rounding=args.rounding,
                  lean_unique=w.interaction, z_bf16=w.interaction and w.compute == "bf16")
    st = fe.stages()
    torch.cuda.synchronize()
    if args.copy_calibration:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters calibrate the
        # counter-measured traffic of the path's kernels
        nb = args.copy_calibration << 20
        src = torch.ones(nb // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    first_main = next(n for n, _ in st if n != "unique")

    def warm():
        if native:
            if pipelined:
                fe.native_start(deep=deep)
            for _ in range(args.warmup):
                fe.step_native(sched)
        elif pipelined:
            fe.pipeline_start()
            for _ in range(args.warmup):
                fe.step_pipelined(fork_after=first_main)
        else:
            for _ in range(args.warmup):
                fe.step()
        torch.cuda.synchronize()

    warm()
    U = int(fe.num_unique.cpu()[0])

    K = args.steps

    # Per-stage durations (diagnostic, before the timed region): each stage alone, bracketed
    # by HIP events on the stream it runs on.
    names = [n for n, _ in st]
    stage_runs = {n: (lambda n=n: fe.run([n])) for n in names}
    evs = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(K)] for n in names}
    for k in range(K):
        for n in names:
            e0, e1 = evs[n][k]
            e0.record()
            stage_runs[n]()
            e1.record()
    torch.cuda.synchronize()
    stage_ms = {n: sum(e0.elapsed_time(e1) for e0, e1 in evs[n]) / K for n in names}
    # The same, cold: before every stage a 1 GiB buffer is written and then read, so that
    # neither the L2s nor the 256 MB MALL hold any of the stage's inputs (or dirty lines).
    stage_ms_cold = None
    if args.cold_steps > 0:
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        cold = {n: [] for n in names}
        for k in range(args.cold_steps):
            for n in names:
                flush.fill_(float(k))
                flush.sum()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                stage_runs[n]()
                e1.record()
                cold[n].append((e0, e1))
        torch.cuda.synchronize()
        stage_ms_cold = {n: sum(a.elapsed_time(b) for a, b in cold[n]) / len(cold[n])
                         for n in names}
        del flush, cold
    byts = stage_bytes(w, U, 8 if fe.src_rows else 16, 2 if fe.z_bf16 else 4)
    # the roofline's kernel: the one that takes the most time per step, among the kernels
    # whose launches the timing marks can bracket (ctr_step_run: the pooling kernel, or the
    # backward's first reduce-by-key level, which carries nearly all of the backward's time)
    markable = ("embbag_fwd", "embbag_bwd_sgd") if native else tuple(SINGLE_KERNEL)
    dominant = max((s for s in stage_ms if s in markable), key=lambda s: stage_ms[s])
    if native:
        fe.native().mark_stage = (ctr.CTR_MARK_BACKWARD if dominant == "embbag_bwd_sgd"
                                  else ctr.CTR_MARK_POOLING)
        warm()
    elif pipelined:
        # the next batch's unique and the stages after the dominant kernel replay from captured
        # graphs (host launch cost); the stages up to the dominant one stay eager so that HIP
        # events on the main stream bracket the dominant kernel itself
        fe.capture_pipelined_parts(fork_after=dominant)
        fe.pipeline_start()
        for _ in range(args.warmup):
            fe.step_pipelined(fork_after=dominant)
        torch.cuda.synchronize()

    # Timed region: K whole steps, bracketed by device synchronizations.  The HIP events
    # dev0[k], dev1[k] bracket step k's pooling kernel on its stream (in graph mode as
    # event-record nodes of the captured steps, so the replay leaves them timed).
    print("[bench] timing %d steps (%s, %s)" % (K, args.launch, "pipelined" if pipelined
                                                else "serial"), file=sys.stderr, flush=True)
    dev0 = [TimingEvent() for _ in range(K)]
    dev1 = [TimingEvent() for _ in range(K)]
    torch.cuda.synchronize()
    if graph:
        g_steps = fe.capture_native(K, sched, [e for pair in zip(dev0, dev1) for e in pair])
        if pipelined:
            fe.native_start(deep=deep)
        g_steps.replay()                 # warm replay
        if pipelined:
            fe.native_start(deep=deep)            # set 0 for the first step (the unique of the step
                                         # before; the graph's last step fills it again)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g_steps.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    else:
        if native:
            def one_step(k):
                fe.step_native(sched, dev0[k], dev1[k])
        else:
            def mark(name, fn):
                if name == dominant:
                    dev0[cur[0]].record()
                    fn()
                    dev1[cur[0]].record()
                else:
                    fn()

            cur = [0]

            def one_step(k):
                cur[0] = k
                if pipelined:
                    fe.step_pipelined(mark, fork_after=dominant)
                else:
                    fe.step(mark)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(K):
            one_step(k)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    dom_ms = sum(dev0[k].elapsed_time(dev1[k]) for k in range(K)) / K
    ms_serial = None
    if pipelined and args.compare_serial:
        # the same K steps with each batch's unique inside its own step, for comparison
        if graph:
            g_ser = fe.capture_native(K, "serial")
            serial_steps = [g_ser.replay]
        else:
            serial_steps = [(lambda: fe.step_native("serial")) if native else fe.step] * K
        for f in serial_steps[:2]:
            f()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for f in serial_steps:
            f()
        torch.cuda.synchronize()
        ms_serial = (time.perf_counter() - t2) * 1e3 / K

    variants = time_variants(fe, w, K) if (w.interaction and args.variants) else None
    if variants is not None and not args.no_cpu:
        print("[bench] CPU oracle of the interaction variants", file=sys.stderr, flush=True)
        cb = cpu_baseline_variants(fe, w, min(args.cpu_seconds, 8.0))
        for name, v in cb.items():
            variants[name]["cpu_baseline"] = v
            variants[name]["samples_per_s"] = w.batch / (variants[name]["ms"] * 1e-3)
    dlrm = None
    if w.interaction and args.dlrm:
        print("[bench] timing the whole DLRM step", file=sys.stderr, flush=True)
        dlrm = time_dlrm(fe, w, K)
        dlrm["mlp_samples_per_s"] = w.batch / (dlrm["mlp_ms"] * 1e-3)
        if not args.no_cpu:
            print("[bench] CPU oracle of the MLPs", file=sys.stderr, flush=True)
            dlrm["cpu_baseline_mlp"] = cpu_baseline_mlp(w, min(args.cpu_seconds, 8.0))

    comp = (compulsory_bytes(w, U, dominant, 2 if fe.z_bf16 else 4) if dominant in ("embbag_fwd", "embbag_bwd_sgd")
            else None)
    step_bytes = sum(byts[k] for k in stage_ms)          # the stages the step runs
    value = w.nnz / (ms_step * 1e-3)
    achieved = byts[dominant] / (dom_ms * 1e-3) / 1e9
    out = {
        "metric": "embedding rows gathered/s + HBM GB/s (fwd+bwd); interaction samples/s",
        "value": value,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "launch": ("hip graph of the K timed steps, captured from ctr_step_run" if graph else
                   "native: one ctr_step_run call enqueues the whole step" if native else
                   "eager up to the dominant kernel, then captured graphs (the next batch's "
                   "unique on a side stream; the rest of the step)" if pipelined else "eager"),
        "schedule": (("pipelined: batch k+1's ID dedup runs during step k on a second stream "
                      "(double-buffered outputs)%s; every call runs once per step"
                      % ({"overlap": "; each backward waits only for its own batch's dedup, "
                                     "so consecutive steps overlap",
                          "overlap2": "; two batches' uniques in flight on two side "
                                      "streams (three output sets), each backward waits only "
                                      "for its own batch's",
                          "early": ", forked when the step starts, joined at its end",
                          "after-pooling": ", forked after the pooling kernel, joined at "
                                           "the step's end"}[args.pipeline] if native
                         else ", forked after the pooling kernel"))
                     if pipelined else "serial: each step dedups its own batch"),
        "ms_per_step_serial": ms_serial if pipelined else ms_step,   # null unless compared
        "z_dtype": "bf16" if fe.z_bf16 else "f32",
        "sorted_src": ("8-byte (row, bag) entries (CTR_SRC_ROWS)" if fe.src_rows else
                       "16-byte (u, bag, key) entries (CTR_SRC_FULL)"),
        "data": "synthetic (seeded; tables from the counter-based fill)",
        "config": {"workload": WORKLOAD_NAMES[args.config] + (
                       "" if args.ids == "zipf" else "; control: uniform IDs, same shapes"),
                   "name": args.config, "ids": args.ids, "rounding": args.rounding,
                   "batch": w.batch, "tables": w.num_tables, "dim": w.dim, "nnz": w.nnz,
                   "unique_rows": U},
        "hbm_gbps_algorithmic": step_bytes / (ms_step * 1e-3) / 1e9,
        "interaction_samples_per_s": (w.batch / ((stage_ms["interaction_fwd"] +
                                                  stage_ms["interaction_bwd"]) * 1e-3)
                                      if w.interaction else None),
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "stage_ms_cold": ({k: round(v, 5) for k, v in stage_ms_cold.items()}
                          if stage_ms_cold else None),
        "variants": variants,
        "dlrm": dlrm,
        "roofline": {"kernel": KERNEL_NAMES.get(dominant, dominant), "stage": dominant,
                     "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(
                         args.config if args.ids == "zipf" else args.config + "_" + args.ids,
                         dominant),
                     "traffic_unit": "bytes per launch leaving L2 toward memory (rocprofv3 TCC_EA0 "
                                     "read requests by size + write requests)",
                     "bytes_per_launch": byts[dominant],
                     "avg_launch_ms": dom_ms,
                     "compulsory_bytes": comp,
                     "compulsory_frac": (comp / (dom_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS
                                         if comp else None),
                     # the kernel alone with cold caches (per-stage timing after a flush)
                     "cold_frac": (byts[dominant] / (stage_ms_cold[dominant] * 1e-3) / 1e9
                                   / HBM_PEAK_GBPS if stage_ms_cold else None)},
        # the pooled gather alone (each stage bracketed by itself before the timed steps):
        # the gather figure, beside the roofline of the kernel that takes the most time
        "pooling": {"ms": round(stage_ms["embbag_fwd"], 5), "bytes": byts["embbag_fwd"],
                    "frac": byts["embbag_fwd"] / (stage_ms["embbag_fwd"] * 1e-3) / 1e9
                    / HBM_PEAK_GBPS,
                    "compulsory_frac": compulsory_bytes(w, U, "embbag_fwd",
                                                        2 if fe.z_bf16 else 4)
                    / (stage_ms["embbag_fwd"] * 1e-3) / 1e9 / HBM_PEAK_GBPS},
        # the interaction alone: memory and matrix-core fractions
        "interaction": interaction_block(w, stage_ms, byts) if w.interaction else None,
    }
    if not args.no_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cb = cpu_baseline(w, args.cpu_seconds)
        out["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        if args.cpu_1thread_seconds > 0 and args.config in ("tiny", "small", "criteo"):
            cb1 = cpu_baseline(w, args.cpu_1thread_seconds, threads=1)
            out["cpu_baseline_1thread"] = {k: cb1[k] for k in ("value", "unit", "cores", "kind",
                                                               "sample")}
    if args.detail:
        det = dict(out)
        det["stage_bytes"] = byts
        det["stage_gbps"] = {k: byts[k] / (stage_ms[k] * 1e-3) / 1e9 for k in stage_ms}
        with open(args.detail, "w") as f:
            json.dump(det, f, indent=1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
