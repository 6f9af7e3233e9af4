"""ctypes wrapper of the plain C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It imports nothing from the
HIP package; callers hand it numpy arrays from the seeded input generator.

Every function returns float64 results together with a magnitude array M (sum of |terms|,
propagated from input magnitudes when given); parity checks use |y_gpu - y| <= rtol * M.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# ORACLE_LIB names another, already built, copy of oracle.c to load instead (a sanitizer
# build, for the host-side tests); build() always makes the default one.
_LOAD = os.environ.get("ORACLE_LIB")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (ISO C11, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
                               "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LOAD:
        lib = ctypes.CDLL(_LOAD)
    else:
        build()
        lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64, u64, f32, f64 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                               ctypes.c_float, ctypes.c_double)
    sig = {
        "orc_set_threads": (None, [ctypes.c_int]),
        "orc_get_threads": (ctypes.c_int, []),
        "orc_round_bf16": (f64, [f64]),
        "orc_round_f32": (f64, [f64]),
        "orc_splitmix64_next": (u64, [P]),
        "orc_table_value": (f64, [u64, i64, i64, i32, i64, i32]),
        "orc_table_rows": (None, [u64, P, i32, i32, i32, P, i64, P]),
        "orc_form_keys": (None, [P, P, i64, i64, P, i64, P]),
        "orc_unique": (i64, [P, i64, P, P, P, P]),
        "orc_gather_rows": (None, [P, u64, P, i32, i32, i32, P, i64, P]),
        "orc_embbag_fwd": (None, [P, u64, P, i32, i32, i32, P, P, i64, P, P]),
        "orc_interaction_fwd": (None, [P, P, i64, i32, i32, i32, P, P]),
        "orc_interaction_bwd": (None, [P, P, P, i64, i32, i32, i32, P, P]),
        "orc_embbag_bwd": (None, [P, P, P, i64, i32, i32, P, i64, P, P]),
        "orc_sparse_sgd": (None, [P, u64, P, i32, i32, i32, P, i64, P, P, f32, P, P]),
        "orc_interaction_self_fwd": (None, [P, P, i64, i32, i32, i32, P, P]),
        "orc_interaction_self_bwd": (None, [P, P, P, i64, i32, i32, i32, P, P]),
        "orc_interaction_gram_fwd": (None, [P, P, i64, i32, i32, i32, P, P]),
        "orc_interaction_gram_bwd": (None, [P, P, P, i64, i32, i32, i32, P, P]),
        "orc_fm_fwd": (None, [P, P, i64, i32, i32, P, P]),
        "orc_fm_bwd": (None, [P, P, P, i64, i32, i32, P, P]),
        "orc_dense_fwd": (None, [P, P, i64, i32, P, P, i32, i32, i32, P, P]),
        "orc_dense_bwd_sgd": (None, [P, i64, i32, P, P, i32, i32, P, P, i32, ctypes.c_double,
                                     P, P, P, P, P, P]),
        "orc_logistic_ne": (None, [P, P, i64, P, P, P, P, P]),
        "orc_dict_lookup": (None, [P, P, P, P, i64, P, i64, P]),
        "orc_dict_pool": (None, [P, u64, i64, i32, i32, P, P, i64, i32, P, P]),
        "orc_sr_bf16": (f64, [f64, ctypes.c_uint32]),
        "orc_round_f16": (f64, [f64]),
        "orc_sr_f16": (f64, [f64, ctypes.c_uint32]),
        "orc_sr_bits": (ctypes.c_uint32, [u64, i64, i64, i32]),
        "orc_sparse_sgd_sr": (None, [P, u64, P, i32, i32, i32, P, i64, P, f32, u64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def get_threads() -> int:
    return int(_load().orc_get_threads())


# ------------------------------------------------------------------------ tables
STYPES = {"f32": 0, "bf16": 1, "f16": 2}      # table storage codes (the C ABI's dtype codes)


class Table:
    """An embedding table as the oracle sees it: either explicit fp32 values
    (``data`` [total_rows, dim]) or the counter-based fill regenerated on demand."""

    def __init__(self, rows: Sequence[int], dim: int, dtype: str, seed: int,
                 data: Optional[np.ndarray] = None):
        self.rows = [int(r) for r in rows]
        self.dim = int(dim)
        self.dtype = dtype
        self.stype = STYPES[dtype]                # storage code: 0 f32, 1 bf16, 2 f16
        self.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
        rb = np.zeros(len(self.rows) + 1, dtype=np.int64)
        rb[1:] = np.cumsum(np.asarray(self.rows, dtype=np.int64))
        self.row_base = rb
        self.data = None if data is None else _c(data, np.float32)

    @property
    def num_tables(self) -> int:
        return len(self.rows)

    @property
    def total_rows(self) -> int:
        return int(self.row_base[-1])

    def args(self):
        return (_p(self.data), self.seed, _p(self.row_base), self.num_tables, self.dim,
                self.stype)


def splitmix64_stream(state: int, count: int) -> list:
    lib = _load()
    st = ctypes.c_uint64(state & 0xFFFFFFFFFFFFFFFF)
    return [int(lib.orc_splitmix64_next(ctypes.byref(st))) for _ in range(count)]


def table_value(seed: int, global_row: int, col: int, dim: int, rows_t: int,
                dtype: str = "f32") -> float:
    return float(_load().orc_table_value(seed & 0xFFFFFFFFFFFFFFFF, global_row, col, dim,
                                         rows_t, STYPES[dtype]))


def round_bf16(x: float) -> float:
    return float(_load().orc_round_bf16(float(x)))


def round_f16(x: float) -> float:
    """x rounded to the nearest IEEE binary16 value, ties to even (as a float)."""
    return float(_load().orc_round_f16(float(x)))


def table_rows(tab: Table, keys: np.ndarray) -> np.ndarray:
    """Stored values of rows ``keys`` (global row ids) as fp32 [len(keys), dim]."""
    keys = _c(keys, np.int64)
    out = np.empty((keys.size, tab.dim), dtype=np.float32)
    _load().orc_table_rows(tab.seed, _p(tab.row_base), tab.num_tables, tab.dim, tab.stype,
                           _p(keys), keys.size, _p(out))
    return out


def full_table(tab: Table) -> np.ndarray:
    return table_rows(tab, np.arange(tab.total_rows, dtype=np.int64))


# ------------------------------------------------------------------------ a1, a2
def form_keys(ids, offsets, num_tables: int, batch: int, row_base=None, modulus: int = 0):
    ids = _c(ids, np.int64)
    offsets = _c(offsets, np.int64)
    rb = None if row_base is None else _c(row_base, np.int64)
    keys = np.empty_like(ids)
    _load().orc_form_keys(_p(ids), _p(offsets), num_tables, batch, _p(rb), int(modulus), _p(keys))
    return keys


def unique(keys):
    """Returns (uniq int64[U], inverse int32[n], perm int32[n], seg int32[U+1])."""
    keys = _c(keys, np.int64)
    n = keys.size
    uniq = np.empty(n, dtype=np.int64)
    inv = np.empty(n, dtype=np.int32)
    perm = np.empty(n, dtype=np.int32)
    seg = np.empty(n + 1, dtype=np.int32)
    U = int(_load().orc_unique(_p(keys), n, _p(uniq), _p(inv), _p(perm), _p(seg)))
    return uniq[:U].copy(), inv, perm, seg[:U + 1].copy()


# ------------------------------------------------------------------------ a3, a4
def gather_rows(tab: Table, rows) -> np.ndarray:
    rows = _c(rows, np.int64)
    out = np.empty((rows.size, tab.dim), dtype=np.float64)
    _load().orc_gather_rows(*tab.args(), _p(rows), rows.size, _p(out))
    return out


def embbag_fwd(tab: Table, ids, offsets, batch: int):
    """Sum-pooled bags: returns (out, mag), each [batch, num_tables, dim] float64.
    ``ids`` are table-local rows; bag (t, b) is offsets[t*batch + b] .. offsets[t*batch+b+1]."""
    ids = _c(ids, np.int64)
    offsets = _c(offsets, np.int64)
    out = np.empty((batch, tab.num_tables, tab.dim), dtype=np.float64)
    mag = np.empty_like(out)
    _load().orc_embbag_fwd(*tab.args(), _p(ids), _p(offsets), batch, _p(out), _p(mag))
    return out, mag


# ------------------------------------------------------------------------ a6, a7
def interaction_fwd(Z, zmag=None, bf16: bool = False):
    """R = [z_0 | <z_i, z_j> for i > j] per sample, with magnitudes.  bf16: every factor of a
    pair product is rounded to bf16 nearest-even first (the products and sums stay exact)."""
    Z = _c(Z, np.float64)
    B, F, d = Z.shape
    zm = None if zmag is None else _c(zmag, np.float64)
    P = F * (F - 1) // 2
    R = np.empty((B, d + P), dtype=np.float64)
    Rm = np.empty_like(R)
    _load().orc_interaction_fwd(_p(Z), _p(zm), B, F, d, int(bool(bf16)), _p(R), _p(Rm))
    return R, Rm


def interaction_bwd(Z, dR, zmag=None, bf16: bool = False):
    """dZ of the strict pair set, with magnitudes.  bf16: the pair gradients and z_j rounded to
    bf16 nearest-even in the products; the dense passthrough's gradient is added as it is."""
    Z = _c(Z, np.float64)
    B, F, d = Z.shape
    dR = _c(dR, np.float64)
    zm = None if zmag is None else _c(zmag, np.float64)
    dZ = np.empty((B, F, d), dtype=np.float64)
    dm = np.empty_like(dZ)
    _load().orc_interaction_bwd(_p(Z), _p(zm), _p(dR), B, F, d, int(bool(bf16)), _p(dZ),
                                _p(dm))
    return dZ, dm


def interaction_self_fwd(Z, zmag=None, bf16: bool = False):
    """Pairs i >= j (self-dots included), P = F(F+1)/2: R = [dense | pairs], with magnitudes."""
    Z = _c(Z, np.float64)
    B, F, d = Z.shape
    zm = None if zmag is None else _c(zmag, np.float64)
    R = np.empty((B, d + F * (F + 1) // 2), dtype=np.float64)
    Rm = np.empty_like(R)
    _load().orc_interaction_self_fwd(_p(Z), _p(zm), B, F, d, int(bool(bf16)), _p(R), _p(Rm))
    return R, Rm


def interaction_self_bwd(Z, dR, zmag=None, bf16: bool = False):
    Z = _c(Z, np.float64)
    B, F, d = Z.shape
    dR = _c(dR, np.float64)
    zm = None if zmag is None else _c(zmag, np.float64)
    dZ = np.empty((B, F, d), dtype=np.float64)
    dm = np.empty_like(dZ)
    _load().orc_interaction_self_bwd(_p(Z), _p(zm), _p(dR), B, F, d, int(bool(bf16)), _p(dZ),
                                     _p(dm))
    return dZ, dm


def interaction_gram_fwd(Z, zmag=None, bf16: bool = False):
    """The whole Gram matrix, P = F^2 row-major: R = [dense | G], with magnitudes."""
    Z = _c(Z, np.float64)
    B, F, d = Z.shape
    zm = None if zmag is None else _c(zmag, np.float64)
    R = np.empty((B, d + F * F), dtype=np.float64)
    Rm = np.empty_like(R)
    _load().orc_interaction_gram_fwd(_p(Z), _p(zm), B, F, d, int(bool(bf16)), _p(R), _p(Rm))
    return R, Rm


def interaction_gram_bwd(Z, dR, zmag=None, bf16: bool = False):
    """dZ of the Gram matrix: dZ_i = sum_j (dG_ij + dG_ji) z_j (+ dense on dZ_0)."""
    Z = _c(Z, np.float64)
    B, F, d = Z.shape
    dR = _c(dR, np.float64)
    zm = None if zmag is None else _c(zmag, np.float64)
    dZ = np.empty((B, F, d), dtype=np.float64)
    dm = np.empty_like(dZ)
    _load().orc_interaction_gram_bwd(_p(Z), _p(zm), _p(dR), B, F, d, int(bool(bf16)), _p(dZ),
                                     _p(dm))
    return dZ, dm


def fm_fwd(Z, zmag=None):
    """Sum of all pair dots per sample (the definition): returns (out [B], mag [B])."""
    Z = _c(Z, np.float64)
    B, F, d = Z.shape
    zm = None if zmag is None else _c(zmag, np.float64)
    out = np.empty(B, dtype=np.float64)
    om = np.empty_like(out)
    _load().orc_fm_fwd(_p(Z), _p(zm), B, F, d, _p(out), _p(om))
    return out, om


def fm_bwd(Z, dout, zmag=None):
    Z = _c(Z, np.float64)
    B, F, d = Z.shape
    dout = _c(dout, np.float64)
    zm = None if zmag is None else _c(zmag, np.float64)
    dZ = np.empty((B, F, d), dtype=np.float64)
    dm = np.empty_like(dZ)
    _load().orc_fm_bwd(_p(Z), _p(zm), _p(dout), B, F, d, _p(dZ), _p(dm))
    return dZ, dm


# ------------------------------------------------------------------------ MLP layers, head
def dense_fwd(X, W, b, relu: bool, bf16: bool, xmag=None):
    """One layer Y = act(X W^T + b): returns (Y, Ym) [M, N] float64.  X [M, K], W [N, K],
    b [N] or None."""
    X = _c(X, np.float64)
    W = _c(W, np.float64)
    M, K = X.shape
    N = W.shape[0]
    assert W.shape[1] == K
    bb = None if b is None else _c(b, np.float64)
    xm = None if xmag is None else _c(xmag, np.float64)
    Y = np.empty((M, N), dtype=np.float64)
    Ym = np.empty_like(Y)
    _load().orc_dense_fwd(_p(X), _p(xm), M, K, _p(W), _p(bb), N, int(bool(relu)),
                          int(bool(bf16)), _p(Y), _p(Ym))
    return Y, Ym


def dense_bwd_sgd(X, W, b, relu: bool, Y, dY, bf16: bool, lr: float, want_dx: bool = True):
    """The layer's backward and SGD step: returns a dict with dX, dXm [M, K] (if want_dx),
    W, Wm [N, K] (updated, binary32 values) and b, bm [N] (if b is not None)."""
    X = _c(X, np.float64)
    W = _c(W, np.float64)
    M, K = X.shape
    N = W.shape[0]
    dY = _c(dY, np.float64)
    Yd = _c(Y if Y is not None else np.zeros((M, N)), np.float64)
    bb = None if b is None else _c(b, np.float64)
    out = {"W": np.empty((N, K)), "Wm": np.empty((N, K))}
    if want_dx:
        out["dX"], out["dXm"] = np.empty((M, K)), np.empty((M, K))
    if bb is not None:
        out["b"], out["bm"] = np.empty(N), np.empty(N)
    _load().orc_dense_bwd_sgd(_p(X), M, K, _p(W), _p(bb), N, int(bool(relu)), _p(Yd), _p(dY),
                              int(bool(bf16)), float(lr), _p(out.get("dX")), _p(out.get("dXm")),
                              _p(out["W"]), _p(out["Wm"]), _p(out.get("b")), _p(out.get("bm")))
    return out


def logistic_ne(s, y):
    """Logistic head: returns (prob, dlogits, dlogits_mag) [M] and (stats, stats_mag) [3],
    stats = [sum ce, sum y, NE]."""
    s = _c(s, np.float64).ravel()
    y = _c(y, np.float64).ravel()
    M = s.size
    prob, dl, dlm = np.empty(M), np.empty(M), np.empty(M)
    st, stm = np.empty(3), np.empty(3)
    _load().orc_logistic_ne(_p(s), _p(y), M, _p(prob), _p(dl), _p(dlm), _p(st), _p(stm))
    return prob, dl, dlm, st, stm


# ------------------------------------------------------------------------ a8, a9
def embbag_bwd(dY, offsets, batch: int, num_tables: int, inverse, U: int, dymag=None):
    """Row gradients per distinct key: returns (g, gmag) [U, dim] float64.
    dY: [batch, num_tables, dim]."""
    dY = _c(dY, np.float64)
    dim = dY.shape[2]
    offsets = _c(offsets, np.int64)
    inverse = _c(inverse, np.int32)
    dym = None if dymag is None else _c(dymag, np.float64)
    g = np.empty((U, dim), dtype=np.float64)
    gm = np.empty_like(g)
    _load().orc_embbag_bwd(_p(dY), _p(dym), _p(offsets), batch, num_tables, dim, _p(inverse),
                           U, _p(g), _p(gm))
    return g, gm


def sparse_sgd(tab: Table, uniq, g, gmag, lr: float):
    """Updated stored values of rows ``uniq``: returns (new_rows, mag) [U, dim] float64."""
    uniq = _c(uniq, np.int64)
    g = _c(g, np.float64)
    gm = _c(gmag, np.float64)
    U = uniq.size
    out = np.empty((U, tab.dim), dtype=np.float64)
    nm = np.empty_like(out)
    _load().orc_sparse_sgd(*tab.args(), _p(uniq), U, _p(g), _p(gm), ctypes.c_float(lr),
                           _p(out), _p(nm))
    return out, nm


def sr_bf16(x: float, r: int) -> float:
    """Stochastic rounding of x to bfloat16 with the 16-bit random integer r."""
    return float(_load().orc_sr_bf16(float(x), int(r) & 0xFFFF))


def sr_bits(seed: int, key: int, col: int, dim: int) -> int:
    """The 16 random bits of element (key, col) of an update drawn with `seed`."""
    return int(_load().orc_sr_bits(seed & 0xFFFFFFFFFFFFFFFF, int(key), int(col), int(dim)))


def sr_f16(x: float, r: int) -> float:
    """Stochastic rounding of x to binary16 with the 16-bit random integer r."""
    return float(_load().orc_sr_f16(float(x), int(r) & 0xFFFF))


def sparse_sgd_sr(tab: Table, uniq, g, lr: float, sr_seed: int):
    """Updated stored values (bf16 or fp16 table) of rows ``uniq`` with stochastic rounding:
    SR(fmaf(-lr, g, w)) per element, g binary32 [U, dim].  Returns float64 [U, dim]."""
    assert tab.stype in (1, 2), "stochastic rounding is defined for 16-bit storage"
    uniq = _c(uniq, np.int64)
    g = _c(g, np.float32)
    U = uniq.size
    out = np.empty((U, tab.dim), dtype=np.float64)
    _load().orc_sparse_sgd_sr(*tab.args(), _p(uniq), U, _p(g), ctypes.c_float(lr),
                              ctypes.c_uint64(sr_seed & 0xFFFFFFFFFFFFFFFF), _p(out))
    return out


def dict_lookup(keys, rows, hot, ids):
    """Values of `ids` in the dictionary (keys, rows, hot): ((hot+1) << 32) | row, or -1."""
    keys = _c(keys, np.int64)
    rows = _c(rows, np.int32)
    hot = None if hot is None else _c(hot, np.int32)
    order = _c(np.argsort(keys, kind="stable"), np.int64)
    ids = _c(ids, np.int64)
    out = np.empty(ids.size, dtype=np.int64)
    _load().orc_dict_lookup(_p(keys), _p(rows), _p(hot), _p(order), keys.size, _p(ids), ids.size,
                            _p(out))
    return out


def dict_pool(tab: "Table", values, offsets, batch: int, num_tables: int):
    """Sum pooling over looked-up values, from the dictionary table `tab` (one table):
    returns (out, mag) [batch, num_tables, dim] float64."""
    assert tab.num_tables == 1
    values = _c(values, np.int64)
    offsets = _c(offsets, np.int64)
    out = np.empty((batch, num_tables, tab.dim), dtype=np.float64)
    om = np.empty_like(out)
    _load().orc_dict_pool(_p(tab.data), tab.seed, tab.total_rows, tab.dim, tab.stype, _p(values),
                          _p(offsets), batch, num_tables, _p(out), _p(om))
    return out, om
