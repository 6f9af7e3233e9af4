"""Seeded synthetic inputs for the sparse front end of a CTR ranking model.

This module only draws random inputs; it performs none of the method's arithmetic
(no keys, no unique, no pooling, no dot products, no gradients).  Both the HIP path
and the CPU oracle consume what it returns, so it must stay free of either.

The workloads stand in for the pages' data, which is not available:
  * "Meta DLRM" (upskillscore.com), section 05: the benchmark draws random synthetic
    categorical features from distributions; the Kaggle ad set has 13 continuous and
    26 categorical features (shape of the Criteo-shaped workload).
  * "How TensorNet Supercharges Sparse Feature Training on TensorFlow", sections
    "Challenges" and "Core Optimizations": ad batches over a near-unbounded ID space.
  * "DHEN" (calwoo.github.io), section 2.1: sparse lookups plus one dense vector.

Embedding-table *values* are not drawn here: both sides fill tables from the same
counter-based definition (splitmix64 of seed XOR (global_row*dim + col), top 24 bits
to a uniform in [0,1), scaled to U(-a, a) with a = fp32(1/sqrt(rows_t))), each with its
own implementation.  This module only states the table shapes and the seed.

Every config draws from ``numpy.random.default_rng(seed)`` in a fixed order, written
out in each builder below.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

TABLE_SEED = 0x5EED_0000_C7A1_0001  # seed of the counter-based table fill


@dataclasses.dataclass
class Workload:
    """One batch of synthetic input for the sparse front end.

    Layouts:
      indices   int64 [nnz]   local row index inside table t (DLRM-style configs), or the
                              raw 64-bit ID (TensorNet config, rows = id mod key_modulus)
      offsets   int64 [T*B+1] CSR bag boundaries, table-major: bag (t, b) is t*B + b
      dense     fp32 [B, d]   the dense ("bottom") vector, slot 0 of Z (None for TensorNet)
      grad_out  fp32          upstream gradient: dR [B, d + P] for DLRM-style configs,
                              dOut [B, slots, d] for the TensorNet config
    """

    name: str
    num_tables: int
    rows: List[int]
    dim: int
    dtype: str                # table storage: "f32", "bf16" or "f16"
    batch: int
    indices: np.ndarray
    offsets: np.ndarray
    dense: Optional[np.ndarray]
    grad_out: np.ndarray
    lr: float
    compute: str              # interaction arithmetic: "f32" or "bf16"
    key_modulus: int = 0      # >0: table row = id mod key_modulus (TensorNet)
    slots: int = 0            # TensorNet: IDs per sample
    table_seed: int = TABLE_SEED
    interaction: bool = True

    @property
    def F(self) -> int:
        return self.num_tables + 1

    @property
    def P(self) -> int:
        return self.F * (self.F - 1) // 2

    @property
    def nnz(self) -> int:
        return int(self.indices.shape[0])

    @property
    def row_base(self) -> np.ndarray:
        rb = np.zeros(len(self.rows) + 1, dtype=np.int64)
        rb[1:] = np.cumsum(np.asarray(self.rows, dtype=np.int64))
        return rb

    @property
    def total_rows(self) -> int:
        return int(sum(self.rows))


# ----------------------------------------------------------------------------- samplers
_CDF_CACHE: Dict[tuple, np.ndarray] = {}


def bounded_zipf(rng: np.random.Generator, alpha: float, n_max: int, size) -> np.ndarray:
    """Draw k in [1, n_max] with P(k) proportional to k^-alpha (inverse-CDF sampling)."""
    key = (float(alpha), int(n_max))
    cdf = _CDF_CACHE.get(key)
    if cdf is None:
        w = np.arange(1, n_max + 1, dtype=np.float64) ** (-alpha)
        cdf = np.cumsum(w)
        cdf /= cdf[-1]
        _CDF_CACHE[key] = cdf
    u = rng.random(size)
    k = np.searchsorted(cdf, u, side="right") + 1
    return np.minimum(k, n_max).astype(np.int64)


def unbounded_zipf_capped(rng: np.random.Generator, alpha: float, cap: int, size: int) -> np.ndarray:
    """Zipf(alpha) ranks on [1, inf) by numpy's sampler, redrawing values above ``cap``."""
    out = rng.zipf(alpha, size).astype(np.int64)
    bad = (out > cap) | (out < 1)
    while bad.any():
        out[bad] = rng.zipf(alpha, int(bad.sum())).astype(np.int64)
        bad = (out > cap) | (out < 1)
    return out


def _offsets_from_lengths(lengths_tb: np.ndarray) -> np.ndarray:
    flat = lengths_tb.reshape(-1).astype(np.int64)
    off = np.zeros(flat.size + 1, dtype=np.int64)
    np.cumsum(flat, out=off[1:])
    return off


# ----------------------------------------------------------------------------- configs
def tiny(seed: int = 0) -> Workload:
    """4 fp32 tables x 1000 rows x d=16, B=128, one uniform ID per table per sample."""
    T, R, d, B = 4, 1000, 16, 128
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, R, size=(T, B), dtype=np.int64)           # draw 1
    offsets = np.arange(T * B + 1, dtype=np.int64)
    dense = rng.standard_normal((B, d)).astype(np.float32)          # draw 2
    F = T + 1
    grad = rng.standard_normal((B, d + F * (F - 1) // 2)).astype(np.float32)  # draw 3
    return Workload("tiny", T, [R] * T, d, "f32", B, idx.reshape(-1), offsets, dense, grad,
                    0.01, "f32")


def _row_ids(rng: np.random.Generator, ids: str, alpha: float, rows: int, size: int) -> np.ndarray:
    """Row indices in [0, rows): bounded Zipf(alpha) ranks minus one, or uniform (the control
    workload with the same shapes, where caches cannot help)."""
    if ids == "uniform":
        return rng.integers(0, rows, size=size, dtype=np.int64)
    return bounded_zipf(rng, alpha, rows, size) - 1


def small(seed: int = 0, batch: int = 2048, rows: int = 1_000_000, ids: str = "zipf") -> Workload:
    """8 fp32 tables x 1M rows x d=64, B=2048, Poisson(20) bags in [1,100], Zipf(1.05) IDs
    (ids="uniform": uniform IDs)."""
    T, d = 8, 64
    rng = np.random.default_rng(seed)
    lengths = np.clip(rng.poisson(20, size=(T, batch)), 1, 100)      # draw 1
    parts = []
    for t in range(T):                                                 # draw 2 (per table)
        parts.append(_row_ids(rng, ids, 1.05, rows, int(lengths[t].sum())))
    idx = np.concatenate(parts)
    dense = rng.standard_normal((batch, d)).astype(np.float32)        # draw 3
    F = T + 1
    grad = rng.standard_normal((batch, d + F * (F - 1) // 2)).astype(np.float32)  # draw 4
    return Workload("small", T, [rows] * T, d, "f32", batch, idx,
                    _offsets_from_lengths(lengths), dense, grad, 0.01, "f32")


def criteo(seed: int = 0, batch: int = 8192, row_scale: float = 1.0, ids: str = "zipf") -> Workload:
    """26 bf16 tables (rows log-uniform in [1e3,1e7]) x d=128, B=8192, 13 log-normal dense
    features projected to 128 by a fixed random matrix; tables 0-12 one-hot, 13-25 bags
    with lengths Zipf(1.1) on [1,64]; IDs Zipf(1.1)."""
    T, d = 26, 128
    rng = np.random.default_rng(seed)
    rows = np.round(10.0 ** rng.uniform(3.0, 7.0, size=T)).astype(np.int64)   # draw 1
    rows = np.maximum(1, np.round(rows * row_scale).astype(np.int64))
    lengths = np.ones((T, batch), dtype=np.int64)
    lengths[13:] = bounded_zipf(rng, 1.1, 64, (T - 13, batch))                 # draw 2
    parts = []
    for t in range(T):                                                          # draw 3
        parts.append(_row_ids(rng, ids, 1.1, int(rows[t]), int(lengths[t].sum())))
    idx = np.concatenate(parts)
    raw = rng.lognormal(0.0, 1.0, size=(batch, 13))                             # draw 4
    proj = rng.normal(0.0, 1.0 / math.sqrt(13.0), size=(13, d))                 # draw 5
    # Fixed random projection of the 13 dense features to d (input preparation on the
    # host, standing in for the bottom MLP, which is not part of the sparse front end).
    dense = (raw @ proj).astype(np.float32)
    F = T + 1
    grad = rng.standard_normal((batch, d + F * (F - 1) // 2)).astype(np.float32)  # draw 6
    return Workload("criteo", T, [int(r) for r in rows], d, "bf16", batch, idx,
                    _offsets_from_lengths(lengths), dense, grad, 0.01, "bf16")


def tensornet(seed: int = 0, batch: int = 65536, slots: int = 100,
              table_rows: int = 20_000_000, key_space: int = 100_000_000_000,
              ids: str = "zipf") -> Workload:
    """65,536 samples x 100 slots of 64-bit IDs, Zipf(1.2) over a 1e11 key space, rows =
    id mod 2e7 of one fp32 table of d=32; one ID per (sample, slot)."""
    d = 32
    rng = np.random.default_rng(seed)
    if ids == "uniform":
        raw = rng.integers(1, key_space + 1, size=batch * slots, dtype=np.int64)  # draw 1
    else:
        raw = unbounded_zipf_capped(rng, 1.2, key_space, batch * slots)       # draw 1
    grad = rng.standard_normal((batch, slots, d)).astype(np.float32)          # draw 2
    # Occurrence i = b*slots + s; every (sample, slot) bag holds exactly one ID.
    offsets = np.arange(batch * slots + 1, dtype=np.int64)
    return Workload("tensornet", 1, [table_rows], d, "f32", batch, raw, offsets, None, grad,
                    0.01, "f32", key_modulus=table_rows, slots=slots, interaction=False)


def large(seed: int = 0, batch: int = 32768, tables: int = 64, rows: int = 4_000_000,
          ids: str = "zipf") -> Workload:
    """64 bf16 tables x 4M rows x d=128, B=32768, Poisson(32) bags in [1,256], Zipf(1.1)
    IDs through a per-table random permutation of the hot ranks."""
    T, d = tables, 128
    rng = np.random.default_rng(seed)
    lengths = np.clip(rng.poisson(32, size=(T, batch)), 1, 256)                # draw 1
    parts = []
    for t in range(T):                                                          # draw 2 (per table)
        if ids == "uniform":
            parts.append(rng.integers(0, rows, size=int(lengths[t].sum()), dtype=np.int64))
            continue
        perm = rng.permutation(rows).astype(np.int64)
        k = bounded_zipf(rng, 1.1, rows, int(lengths[t].sum()))
        parts.append(perm[k - 1])
    idx = np.concatenate(parts)
    dense = rng.standard_normal((batch, d)).astype(np.float32)                  # draw 3
    F = T + 1
    grad = rng.standard_normal((batch, d + F * (F - 1) // 2)).astype(np.float32)  # draw 4
    return Workload("large", T, [rows] * T, d, "bf16", batch, idx,
                    _offsets_from_lengths(lengths), dense, grad, 0.01, "bf16")


@dataclasses.dataclass
class DictWorkload:
    """Inference-side lookup from an exported sparse-embedding dictionary ("How TensorNet
    Supercharges Sparse Feature Training on TensorFlow", "Inference Optimization": online
    inference reads a pre-exported sparse embedding dictionary) with a hot-row HBM cache in
    front of it (the HBM tier of a hierarchical GPU parameter server, "Tera-scale training"
    review, hardware-aware framework figure).

    Ranks r = 1, 2, ... order IDs by popularity; rank r has the raw 64-bit ID
    key_of_rank(r), a fixed affine bijection of [1, key_space].  The dictionary holds ranks
    1..N: dict_keys[r-1] = key_of_rank(r), stored at row dict_rows[r-1] of a table of N rows
    (a random permutation), and ranks 1..H also sit in the HBM cache, at slot r - 1
    (hot_slots; -1 for the others).  A query ID has a Zipf(alpha) rank over the key space,
    so ranks above N miss the dictionary.  One ID per (sample, slot) bag."""

    name: str
    dim: int
    dtype: str
    batch: int
    slots: int
    key_space: int
    dict_keys: np.ndarray        # int64 [N]
    dict_rows: np.ndarray        # int32 [N]
    hot_slots: np.ndarray        # int32 [N]
    hot: int                     # H
    indices: np.ndarray          # int64 [batch * slots] raw query IDs
    offsets: np.ndarray          # int64 [batch * slots + 1]
    table_seed: int = TABLE_SEED

    @property
    def entries(self) -> int:
        return int(self.dict_keys.shape[0])

    @property
    def nnz(self) -> int:
        return int(self.indices.shape[0])


_KEY_MULT = 38_196_601_123       # odd and not a multiple of 5: coprime to 10^11
_KEY_ADD = 12_345_678_901


def key_of_rank(r: np.ndarray, key_space: int) -> np.ndarray:
    """A fixed bijection of [1, key_space] (key_space = 10^11): ((r-1)*M + A) mod key_space + 1."""
    r = np.asarray(r, dtype=object) if key_space > (1 << 31) else np.asarray(r)
    k = ((r - 1) * _KEY_MULT + _KEY_ADD) % key_space + 1
    return np.asarray(k, dtype=np.int64)


def dictionary(seed: int = 0, batch: int = 65536, slots: int = 100, entries: int = 20_000_000,
               hot: int = 2_000_000, key_space: int = 100_000_000_000,
               alpha: float = 1.2) -> DictWorkload:
    """The TensorNet batch shape (65,536 x 100 IDs, Zipf(1.2) over 1e11) against a dictionary
    of the 2e7 most popular IDs (d = 32 fp32), the 2e6 hottest also cached in HBM."""
    rng = np.random.default_rng(seed)
    ranks = np.arange(1, entries + 1, dtype=np.int64)
    keys = _affine_keys(ranks, key_space)
    rows = rng.permutation(entries).astype(np.int32)                           # draw 1
    hot_slots = np.full(entries, -1, dtype=np.int32)
    hot_slots[:hot] = np.arange(hot, dtype=np.int32)
    q = unbounded_zipf_capped(rng, alpha, key_space, batch * slots)            # draw 2
    return DictWorkload("dictionary", 32, "f32", batch, slots, key_space, keys, rows,
                        hot_slots, hot, _affine_keys(q, key_space),
                        np.arange(batch * slots + 1, dtype=np.int64))


def _affine_keys(ranks: np.ndarray, key_space: int) -> np.ndarray:
    """key_of_rank without object arrays: (r-1)*M mod key_space by 32-bit halves of M."""
    r = (np.asarray(ranks, dtype=np.int64) - 1) % key_space
    lo, hi = _KEY_MULT & 0xFFFFFFFF, _KEY_MULT >> 32
    # (r * (hi*2^32 + lo)) mod K = ((r*hi mod K) * 2^32 + r*lo) mod K, each product < 2^63
    a = (r * hi) % key_space
    a = ((a * (1 << 16)) % key_space * (1 << 16)) % key_space
    b = ((r % key_space) * lo) % key_space if lo < (1 << 26) else _mulmod(r, lo, key_space)
    return ((a + b + _KEY_ADD) % key_space + 1).astype(np.int64)


def _mulmod(r: np.ndarray, m: int, k: int) -> np.ndarray:
    """(r * m) mod k for r < k < 2^37 and m < 2^32, without overflow: m in 16-bit halves."""
    m_lo, m_hi = m & 0xFFFF, m >> 16
    a = (r * m_hi) % k
    a = (a * (1 << 16)) % k
    return (a + (r * m_lo) % k) % k


def slice_batch(w: Workload, b: int) -> Workload:
    """The first `b` samples of every table (a bounded sample of the same batch)."""
    b = min(int(b), w.batch)
    if not w.interaction:                        # one occurrence per (sample, slot)
        n = b * w.slots
        return dataclasses.replace(w, batch=b, indices=w.indices[:n],
                                   offsets=np.arange(n + 1, dtype=np.int64),
                                   grad_out=w.grad_out[:b])
    T, B = w.num_tables, w.batch
    parts, lens = [], []
    for t in range(T):
        lo, hi = int(w.offsets[t * B]), int(w.offsets[t * B + b])
        parts.append(w.indices[lo:hi])
        lens.append(np.diff(w.offsets[t * B:t * B + b + 1]))
    off = np.zeros(T * b + 1, dtype=np.int64)
    np.cumsum(np.concatenate(lens), out=off[1:])
    return dataclasses.replace(w, batch=b, indices=np.concatenate(parts), offsets=off,
                               dense=w.dense[:b], grad_out=w.grad_out[:b])


BUILDERS = {"tiny": tiny, "small": small, "criteo": criteo, "tensornet": tensornet,
            "large": large}


def make(name: str, **kw) -> Workload:
    return BUILDERS[name](**kw)


# ----------------------------------------------------------------------------- DLRM step
DLRM_BOTTOM = (512, 256)            # hidden widths of the bottom MLP (output: the dim)
DLRM_TOP = (1024, 1024, 512, 256)   # hidden widths of the top MLP (output: one logit)
DLRM_DENSE = 13                     # continuous features per sample
DLRM_CLICK_RATE = 0.25


@dataclasses.dataclass
class DlrmInputs:
    """Inputs of a whole DLRM training step beside the sparse batch: continuous features,
    click labels, and the initial MLP parameters (W [out, in], b [out]) per layer."""

    dense_raw: np.ndarray           # fp32 [B, n_dense]
    labels: np.ndarray              # fp32 [B], 0 or 1
    bottom: List[tuple]             # [(W, b)], widths n_dense -> ... -> dim
    top: List[tuple]                # [(W, b)], widths dim + P -> ... -> 1


def dlrm_inputs(w: Workload, seed: int = 0, n_dense: int = DLRM_DENSE,
                bottom=DLRM_BOTTOM, top=DLRM_TOP,
                click_rate: float = DLRM_CLICK_RATE) -> DlrmInputs:
    """Continuous features log-normal(0, 1), labels Bernoulli(click_rate), every weight and
    bias U(-1/sqrt(fan_in), 1/sqrt(fan_in)); draws in that order, layers bottom to top."""
    assert w.interaction
    rng = np.random.default_rng(seed + 77)
    B = w.batch
    raw = rng.lognormal(0.0, 1.0, size=(B, n_dense)).astype(np.float32)
    labels = (rng.random(B) < click_rate).astype(np.float32)

    def mlp(widths):
        layers = []
        for fi, fo in zip(widths[:-1], widths[1:]):
            a = np.float32(1.0 / math.sqrt(fi))
            W = (rng.uniform(-1.0, 1.0, size=(fo, fi)).astype(np.float32) * a)
            b = (rng.uniform(-1.0, 1.0, size=fo).astype(np.float32) * a)
            layers.append((W, b))
        return layers

    return DlrmInputs(raw, labels, mlp([n_dense, *bottom, w.dim]),
                      mlp([w.dim + w.P, *top, 1]))
