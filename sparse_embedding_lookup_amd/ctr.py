"""Thin Python binding of libctr (include/ctr.h), one function per C entry point, same names.

Only argument marshalling happens here: torch tensors provide device memory and the current
stream, every step of the computation runs in the HIP kernels of libctr.so.  There is no CPU
fallback: if the library is missing or fails to load, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# CTR_LIB names another build of the library (a sanitizer build of its host code, for the
# host-side tests); the default is the in-tree libctr.so.  A missing library always raises.
LIB_PATH = os.environ.get("CTR_LIB") or os.path.join(_HERE, "libctr.so")

CTR_OK, CTR_ERR_INVALID_ARGUMENT, CTR_ERR_UNSUPPORTED, CTR_ERR_WORKSPACE_TOO_SMALL, CTR_ERR_HIP = range(5)
CTR_F32, CTR_BF16, CTR_F16 = 0, 1, 2
CTR_I32, CTR_I64 = 0, 1

EXPORTED = [
    "ctr_version", "ctr_status_string", "ctr_last_error_message", "ctr_unique_ids",
    "ctr_gather_rows",
    "ctr_embbag_fwd", "ctr_embbag_bwd", "ctr_embbag_bwd_sgd", "ctr_sparse_sgd",
    "ctr_dot_interaction_fwd",
    "ctr_dot_interaction_bwd", "ctr_init_tables_hash", "ctr_validate_csr", "ctr_step_run",
    "ctr_step_unique", "ctr_sr_step_seed",
    "ctr_dot_interaction_self_fwd", "ctr_dot_interaction_self_bwd", "ctr_fm_interaction_fwd",
    "ctr_fm_interaction_bwd", "ctr_dict_build", "ctr_dict_lookup", "ctr_dict_embbag_fwd",
    "ctr_step_run_deep",
    "ctr_dense_fwd", "ctr_dense_bwd_sgd", "ctr_logistic_ne", "ctr_embbag_interaction_fwd",
    "ctr_embbag_bwd_sgd_noalloc", "ctr_embbag_bwd_noalloc_scratch_bytes",
    "ctr_noalloc_scratch_capacity", "ctr_dot_interaction_gram_fwd",
    "ctr_dot_interaction_gram_bwd",
]

CTR_STEP_POOLED_INTERACTION, CTR_STEP_BATCH_MATRIX = 0, 1
CTR_SCHEDULE_SERIAL, CTR_SCHEDULE_PIPELINED, CTR_SCHEDULE_PIPELINED_EARLY = 0, 1, 2
CTR_SCHEDULE_PIPELINED_OVERLAP = 3
CTR_ROUND_NEAREST, CTR_ROUND_STOCHASTIC = 0, 1
CTR_MARK_POOLING, CTR_MARK_BACKWARD = 0, 1
CTR_SRC_FULL, CTR_SRC_ROWS = 0, 1


class CtrStep(ctypes.Structure):
    """ctr_step_t of include/ctr.h: every device buffer of one training step."""
    _P = ctypes.c_void_p
    _fields_ = [("kind", ctypes.c_int32), ("index_type", ctypes.c_int32), ("indices", _P),
                ("nnz", ctypes.c_int64), ("offsets", _P), ("batch", ctypes.c_int64),
                ("num_tables", ctypes.c_int32), ("dim", ctypes.c_int32), ("row_base", _P),
                ("key_modulus", ctypes.c_int64), ("table", _P), ("dtype", ctypes.c_int32),
                ("compute", ctypes.c_int32), ("total_rows", ctypes.c_int64),
                ("lr", ctypes.c_float), ("Z", _P), ("R", _P), ("dR", _P), ("dZ", _P), ("E", _P),
                ("out", _P), ("dout", _P), ("row_grads", _P), ("ws_unique", _P),
                ("ws_unique_bytes", ctypes.c_size_t), ("ws_bwd", _P),
                ("ws_bwd_bytes", ctypes.c_size_t), ("uniq", _P * 3), ("inverse", _P * 3),
                ("num_unique", _P * 3), ("perm", _P * 3), ("seg_offsets", _P * 3),
                ("sorted_src", _P * 3), ("rounding", ctypes.c_int32),
                ("sr_seed", ctypes.c_uint64), ("grad_dtype", ctypes.c_int32),
                ("ws_unique2", _P), ("ws_unique2_bytes", ctypes.c_size_t),
                ("mark_stage", ctypes.c_int32), ("max_table_rows", ctypes.c_int64),
                ("ws_pool", _P), ("ws_pool_bytes", ctypes.c_size_t),
                ("src_layout", ctypes.c_int32), ("z_dtype", ctypes.c_int32)]

_lib = None


class CtrError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s failed: %s (%s)" % (fn, _status_name(status), msg))
        self.status = status


def _status_name(s: int) -> str:
    return ["CTR_OK", "CTR_ERR_INVALID_ARGUMENT", "CTR_ERR_UNSUPPORTED",
            "CTR_ERR_WORKSPACE_TOO_SMALL", "CTR_ERR_HIP"][s] if 0 <= s < 5 else "CTR_ERR_UNKNOWN"


def load() -> ctypes.CDLL:
    """Loads libctr.so from the package directory (built by build.py); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libctr.so is not built (run python -m sparse_embedding_lookup_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, u64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                 ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t)
    PS = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "ctr_version": (i32, []),
        "ctr_status_string": (ctypes.c_char_p, [i32]),
        "ctr_last_error_message": (ctypes.c_char_p, []),
        "ctr_unique_ids": (i32, [P, i32, i64, P, i64, i32, P, i64, i64, i64, P, P, P, P, P, P,
                                 i32, P, PS, P]),
        "ctr_gather_rows": (i32, [P, i32, i64, i32, P, P, i64, P, P]),
        "ctr_embbag_fwd": (i32, [P, i32, i64, i32, P, i32, P, i32, i64, P, i64, P, i32, i64, i64,
                                 P, PS, P]),
        "ctr_embbag_bwd": (i32, [P, i64, i64, P, i64, i32, i32, i64, P, P, P, P, P, P, PS, P]),
        "ctr_embbag_bwd_sgd": (i32, [P, i32, i64, i64, P, i64, i32, i64, P, i32, P, P, i32, i64,
                                     i32, P, f32, i32, u64, P, P, PS, P]),
        "ctr_sparse_sgd": (i32, [P, i32, i64, i32, P, P, i64, P, f32, i32, u64, P]),
        "ctr_sr_step_seed": (u64, [u64, i64]),
        "ctr_dot_interaction_self_fwd": (i32, [P, i64, i32, i32, i32, P, i64, P]),
        "ctr_dot_interaction_self_bwd": (i32, [P, P, i64, i64, i32, i32, i32, i32, P, P]),
        "ctr_dot_interaction_gram_fwd": (i32, [P, i64, i32, i32, i32, P, i64, P]),
        "ctr_dot_interaction_gram_bwd": (i32, [P, P, i64, i64, i32, i32, i32, i32, P, P]),
        "ctr_fm_interaction_fwd": (i32, [P, i64, i32, i32, P, P]),
        "ctr_fm_interaction_bwd": (i32, [P, P, i64, i32, i32, P, P]),
        "ctr_embbag_bwd_sgd_noalloc": (i32, [P, i32, i64, i64, P, i64, i32, i64, P, i32, P, P,
                                             i32, i64, i32, P, f32, i32, u64, P, P]),
        "ctr_embbag_bwd_noalloc_scratch_bytes": (sz, [i64, i32]),
        "ctr_noalloc_scratch_capacity": (sz, []),
        "ctr_dict_build": (i32, [P, P, P, i64, P, i64, P, P]),
        "ctr_dict_lookup": (i32, [P, i64, P, i64, P, P]),
        "ctr_dict_embbag_fwd": (i32, [P, i64, P, i64, i32, P, i64, P, i64, i32, i32, P, i64,
                                      i64, P]),
        "ctr_dot_interaction_fwd": (i32, [P, i32, i64, i32, i32, i32, P, i64, P]),
        "ctr_embbag_interaction_fwd": (i32, [P, i32, i64, i32, P, i32, P, i32, i64, P, i64, P,
                                             i32, P, i64, P]),
        "ctr_dot_interaction_bwd": (i32, [P, i32, P, i64, i64, i32, i32, i32, i32, P, P]),
        "ctr_init_tables_hash": (i32, [P, i32, i32, P, i32, u64, P]),
        "ctr_validate_csr": (i32, [P, i32, i64, P, i64, i32, P, i64, P, P]),
        "ctr_step_run": (i32, [P, i64, i32, P, P, P, P, P, P]),
        "ctr_step_unique": (i32, [P, i32, P]),
        "ctr_step_run_deep": (i32, [P, i64, P, P, P, P, P, P]),
        "ctr_dense_fwd": (i32, [P, i64, i64, i32, P, P, i32, i32, i32, P, i64, P]),
        "ctr_dense_bwd_sgd": (i32, [P, i64, i64, i32, P, P, i32, i32, P, i64, P, i32, i64, i32,
                                    f32, P, i64, P, PS, P]),
        "ctr_logistic_ne": (i32, [P, i64, P, i64, P, P, i64, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _require_f32(Z: torch.Tensor, fn: str) -> None:
    """The entry points whose Z is fp32 only (their C signature carries no Z type)."""
    if Z.dtype != torch.float32:
        raise TypeError("%s takes an fp32 Z, not %s" % (fn, Z.dtype))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def src_layout(sorted_src: Optional[torch.Tensor]) -> int:
    """The layout code of a sorted_src tensor: int32 [n, 4] quadruples (CTR_SRC_FULL) or
    [n, 2] row entries (CTR_SRC_ROWS)."""
    if sorted_src is None or sorted_src.shape[-1] == 4:
        return CTR_SRC_FULL
    if sorted_src.shape[-1] == 2:
        return CTR_SRC_ROWS
    raise ValueError("sorted_src must be int32 [n, 4] or [n, 2], not %s" % (tuple(sorted_src.shape),))


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, status: int) -> None:
    if status != CTR_OK:
        raise CtrError(fn, status, load().ctr_last_error_message().decode())


class Call:
    """A libctr call whose arguments were marshalled once; calling it only reads the current
    stream (so it also works under stream capture) and checks the status."""
    __slots__ = ("name", "fn", "args", "result")

    def __init__(self, name: str, args: tuple, result=None):
        self.name = name
        self.fn = getattr(load(), name)
        self.args = args
        self.result = result

    def __call__(self, stream=None):
        st = self.fn(*self.args, _stream(stream))
        if st != CTR_OK:
            _check(self.name, st)
        return self.result


def _run(name: str, args: tuple, stream, prepare: bool, result=None):
    call = Call(name, args, result)
    return call if prepare else call(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CTR_F32
    if t.dtype == torch.bfloat16:
        return CTR_BF16
    if t.dtype == torch.float16:
        return CTR_F16
    raise TypeError("dtype must be float32, bfloat16 or float16")


def _index_code(t: torch.Tensor) -> int:
    if t.dtype == torch.int64:
        return CTR_I64
    if t.dtype == torch.int32:
        return CTR_I32
    raise TypeError("index dtype must be int32 or int64")


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def unique_workspace_bytes(n: int) -> int:
    """Workspace of ctr_unique_ids for n occurrences (the library's two-call query)."""
    wsb = ctypes.c_size_t(0)
    _check("ctr_unique_ids", load().ctr_unique_ids(None, CTR_I64, n, None, 0, 0, None, 0, 0, 0,
                                                   None, None, None, None, None, None,
                                                   CTR_SRC_FULL, None, ctypes.byref(wsb), None))
    return wsb.value


def embbag_bwd_workspace_bytes(nnz: int, dim: int) -> int:
    """Workspace of ctr_embbag_bwd (the library's two-call query)."""
    wsb = ctypes.c_size_t(0)
    _check("ctr_embbag_bwd", load().ctr_embbag_bwd(None, 0, 0, None, 1, 1, dim, nnz, None, None,
                                                   None, None, None, None, ctypes.byref(wsb),
                                                   None))
    return wsb.value


# ----------------------------------------------------------------------------- entry points
def ctr_version() -> int:
    return int(load().ctr_version())


def ctr_unique_ids(ids: torch.Tensor, *, offsets: Optional[torch.Tensor] = None, batch: int = 0,
                   num_tables: int = 0, row_base: Optional[torch.Tensor] = None,
                   total_rows: int = 0, max_table_rows: int = 0, key_modulus: int = 0,
                   want_perm: bool = True,
                   want_seg: bool = True, want_inverse: bool = True,
                   workspace: Optional[torch.Tensor] = None,
                   out: Optional[tuple] = None, sorted_src: Optional[torch.Tensor] = None,
                   stream=None, prepare: bool = False
                   ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, Optional[torch.Tensor],
                              Optional[torch.Tensor]]:
    """Returns (uniq int64[n], inverse int32[n], num_unique int32[1], perm, seg_offsets);
    only the first num_unique entries of uniq (and num_unique+1 of seg_offsets) are set.
    ``out`` may supply those five tensors (inverse / perm / seg_offsets may be None: the
    library then leaves them out, and the sort carries no occurrence payload when none of
    the three is asked for and the bags ride along); ``sorted_src``
    (int32 [n, 4], 16-byte aligned) receives (distinct-row index, bag, key low word, key high
    word) for every sorted position, or as int32 [n, 2] (8-byte aligned) the row entries
    (key, bag) of CTR_SRC_ROWS."""
    n = ids.numel()
    dev = ids.device
    if out is not None:
        uniq, inv, nu, perm, seg = out
    else:
        uniq = torch.empty(max(n, 1), dtype=torch.int64, device=dev)
        inv = torch.empty(max(n, 1), dtype=torch.int32, device=dev) if want_inverse else None
        nu = torch.empty(1, dtype=torch.int32, device=dev)
        perm = torch.empty(max(n, 1), dtype=torch.int32, device=dev) if want_perm else None
        seg = torch.empty(n + 1, dtype=torch.int32, device=dev) if want_seg else None
    args = (_ptr(ids), _index_code(ids), n, _ptr(offsets), batch, num_tables, _ptr(row_base),
            total_rows, max_table_rows, key_modulus)
    if workspace is None:
        workspace = _workspace(unique_workspace_bytes(n), dev)
    ws = workspace
    wsb = ctypes.c_size_t(ws.numel())
    full = args + (_ptr(uniq), _ptr(inv), _ptr(nu), _ptr(perm), _ptr(seg), _ptr(sorted_src),
                   src_layout(sorted_src), _ptr(ws), ctypes.byref(wsb))
    res = (uniq[:n], (inv[:n] if inv is not None else None), nu,
           (perm[:n] if perm is not None else None), seg)
    return _run("ctr_unique_ids", full, stream, prepare, res)


def ctr_gather_rows(table: torch.Tensor, rows: torch.Tensor, num_rows: torch.Tensor,
                    capacity: int, out: Optional[torch.Tensor] = None, stream=None,
                    prepare: bool = False):
    total_rows, dim = table.shape
    if out is None:
        out = torch.empty((max(capacity, 1), dim), dtype=torch.float32, device=table.device)
    args = (_ptr(table), _dtype_code(table), total_rows, dim, _ptr(rows), _ptr(num_rows),
            capacity, _ptr(out))
    return _run("ctr_gather_rows", args, stream, prepare, out)


def embbag_fwd_workspace_bytes(nnz: int, dim: int) -> int:
    """Workspace of ctr_embbag_fwd (the library's two-call query)."""
    wsb = ctypes.c_size_t(0)
    _check("ctr_embbag_fwd", load().ctr_embbag_fwd(None, CTR_F32, 0, dim, None, 1, None, CTR_I64,
                                                   nnz, None, 0, None, CTR_F32, 0, 0, None,
                                                   ctypes.byref(wsb), None))
    return wsb.value


def ctr_embbag_fwd(table: torch.Tensor, indices: torch.Tensor, offsets: torch.Tensor,
                   batch: int, num_tables: int, out: torch.Tensor, out_stride_b: int,
                   out_stride_t: int, row_base: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None,
                   prepare: bool = False):
    """Sum pooling of the bags into out (fp32, or bf16: the fp32 sums rounded once at the
    store); ``workspace`` (uint8, from embbag_fwd_workspace_bytes) holds the partial sums of
    bags longer than 4096 occurrences (allocated when None)."""
    total_rows, dim = table.shape
    nnz = indices.numel()
    if workspace is None:
        workspace = _workspace(embbag_fwd_workspace_bytes(nnz, dim), table.device)
    wsb = ctypes.c_size_t(workspace.numel())
    args = (_ptr(table), _dtype_code(table), total_rows, dim, _ptr(row_base), num_tables,
            _ptr(indices), _index_code(indices), nnz, _ptr(offsets), batch, _ptr(out),
            _dtype_code(out), out_stride_b, out_stride_t, _ptr(workspace), ctypes.byref(wsb))
    return _run("ctr_embbag_fwd", args, stream, prepare, out)


def ctr_embbag_bwd(grad: torch.Tensor, grad_stride_b: int, grad_stride_t: int,
                   offsets: torch.Tensor, batch: int, num_tables: int, dim: int,
                   perm: Optional[torch.Tensor], inverse: Optional[torch.Tensor],
                   num_unique: torch.Tensor, row_grads: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None,
                   sorted_src: Optional[torch.Tensor] = None, nnz: Optional[int] = None,
                   stream=None, prepare: bool = False):
    """Per-row gradient sums; the grouping comes from ``sorted_src`` or from (perm, inverse).
    A bf16 ``grad`` (summed in fp32) needs ``sorted_src``."""
    if nnz is None:
        nnz = sorted_src.shape[0] if sorted_src is not None else perm.numel()
    dev = grad.device
    if row_grads is None:
        row_grads = torch.empty((max(nnz, 1), dim), dtype=torch.float32, device=dev)
    if grad.dtype == torch.bfloat16:
        if workspace is None:
            workspace = _workspace(embbag_bwd_workspace_bytes(nnz, dim), dev)
        return ctr_embbag_bwd_sgd(grad, grad_stride_b, grad_stride_t, offsets, batch,
                                  num_tables, nnz, sorted_src, num_unique, None, None, 0.0,
                                  row_grads=row_grads, workspace=workspace, dim=dim,
                                  stream=stream, prepare=prepare)
    args = (_ptr(grad), grad_stride_b, grad_stride_t, _ptr(offsets), batch, num_tables, dim, nnz,
            _ptr(perm), _ptr(inverse), _ptr(sorted_src), _ptr(num_unique), _ptr(row_grads))
    if workspace is None:
        workspace = _workspace(embbag_bwd_workspace_bytes(nnz, dim), dev)
    ws = workspace
    wsb = ctypes.c_size_t(ws.numel())
    return _run("ctr_embbag_bwd", args + (_ptr(ws), ctypes.byref(wsb)), stream, prepare,
                row_grads)


def ctr_embbag_bwd_sgd(grad: torch.Tensor, grad_stride_b: int, grad_stride_t: int,
                       offsets: torch.Tensor, batch: int, num_tables: int, nnz: int,
                       sorted_src: torch.Tensor, num_unique: torch.Tensor,
                       table: Optional[torch.Tensor], uniq: Optional[torch.Tensor], lr: float,
                       row_grads: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None,
                       rounding: int = CTR_ROUND_NEAREST, seed: int = 0, dim: int = 0,
                       stream=None, prepare: bool = False):
    """Per-row gradient sums applied straight to the table as the sparse SGD update, rounded
    by ``rounding`` (stochastic: random bits from ``seed``).  The gradient type is the
    tensor's (fp32 or bf16); table None: row sums into row_grads only (dim then required).
    ``sorted_src`` of shape [n, 2] holds row entries (CTR_SRC_ROWS: uniq unused, no
    row_grads)."""
    total_rows, d = (0, dim) if table is None else table.shape
    if workspace is None:
        workspace = _workspace(embbag_bwd_workspace_bytes(nnz, d), grad.device)
    wsb = ctypes.c_size_t(workspace.numel())
    args = (_ptr(grad), _dtype_code(grad), grad_stride_b, grad_stride_t, _ptr(offsets), batch,
            num_tables, nnz, _ptr(sorted_src), src_layout(sorted_src), _ptr(num_unique),
            _ptr(table), CTR_F32 if table is None else _dtype_code(table), total_rows, d,
            _ptr(uniq), ctypes.c_float(lr), rounding,
            ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), _ptr(row_grads), _ptr(workspace),
            ctypes.byref(wsb))
    return _run("ctr_embbag_bwd_sgd", args, stream, prepare, row_grads)


def ctr_embbag_bwd_sgd_noalloc(grad: torch.Tensor, grad_stride_b: int, grad_stride_t: int,
                               offsets: torch.Tensor, batch: int, num_tables: int, nnz: int,
                               sorted_src: torch.Tensor, num_unique: torch.Tensor,
                               table: Optional[torch.Tensor], uniq: Optional[torch.Tensor],
                               lr: float, row_grads: Optional[torch.Tensor] = None,
                               rounding: int = CTR_ROUND_NEAREST, seed: int = 0, dim: int = 0,
                               stream=None, prepare: bool = False):
    """ctr_embbag_bwd_sgd without a workspace: the library's per-GPU scratch holds the
    reduce-by-key carries (table None: row sums into row_grads only; dim then required)."""
    total_rows, d = (0, dim) if table is None else table.shape
    args = (_ptr(grad), _dtype_code(grad), grad_stride_b, grad_stride_t, _ptr(offsets), batch,
            num_tables, nnz, _ptr(sorted_src), src_layout(sorted_src), _ptr(num_unique),
            _ptr(table), CTR_F32 if table is None else _dtype_code(table), total_rows, d,
            _ptr(uniq), ctypes.c_float(lr), rounding,
            ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), _ptr(row_grads))
    return _run("ctr_embbag_bwd_sgd_noalloc", args, stream, prepare, row_grads)


def noalloc_scratch_bytes(nnz: int, dim: int) -> int:
    return int(load().ctr_embbag_bwd_noalloc_scratch_bytes(nnz, dim))


def noalloc_scratch_capacity() -> int:
    return int(load().ctr_noalloc_scratch_capacity())


def ctr_sr_step_seed(base: int, k: int) -> int:
    """Seed of the k-th stochastically rounded update of a run seeded with base."""
    return int(load().ctr_sr_step_seed(base & 0xFFFFFFFFFFFFFFFF, k))


def ctr_sparse_sgd(table: torch.Tensor, uniq: torch.Tensor, num_unique: torch.Tensor,
                   capacity: int, row_grads: torch.Tensor, lr: float,
                   rounding: int = CTR_ROUND_NEAREST, seed: int = 0, stream=None,
                   prepare: bool = False):
    """Update of the touched rows, rounded by ``rounding`` (stochastic: bf16 table, random
    bits from ``seed``)."""
    total_rows, dim = table.shape
    args = (_ptr(table), _dtype_code(table), total_rows, dim, _ptr(uniq), _ptr(num_unique),
            capacity, _ptr(row_grads), ctypes.c_float(lr), rounding,
            ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF))
    return _run("ctr_sparse_sgd", args, stream, prepare)


def ctr_dot_interaction_fwd(Z: torch.Tensor, compute: int = CTR_F32,
                            R: Optional[torch.Tensor] = None, stream=None,
                            prepare: bool = False):
    B, F, d = Z.shape
    P = F * (F - 1) // 2
    if R is None:
        R = torch.empty((B, d + P), dtype=torch.float32, device=Z.device)
    args = (_ptr(Z), _dtype_code(Z), B, F, d, compute, _ptr(R), R.stride(0))
    return _run("ctr_dot_interaction_fwd", args, stream, prepare, R)


def ctr_embbag_interaction_fwd(table: torch.Tensor, indices: torch.Tensor,
                               offsets: torch.Tensor, Z: torch.Tensor, compute: int = CTR_F32,
                               R: Optional[torch.Tensor] = None,
                               row_base: Optional[torch.Tensor] = None, stream=None,
                               prepare: bool = False):
    """Pooling into Z[:, 1:, :] and the dot interaction of Z into R in one call; Z[:, 0, :]
    (the dense vectors) is an input."""
    total_rows, dim = table.shape
    B, F, d = Z.shape
    _require_f32(Z, "ctr_embbag_interaction_fwd")
    assert d == dim and Z.is_contiguous()
    P = F * (F - 1) // 2
    if R is None:
        R = torch.empty((B, d + P), dtype=torch.float32, device=Z.device)
    args = (_ptr(table), _dtype_code(table), total_rows, dim, _ptr(row_base), F - 1,
            _ptr(indices), _index_code(indices), indices.numel(), _ptr(offsets), B, _ptr(Z),
            compute, _ptr(R), R.stride(0))
    return _run("ctr_embbag_interaction_fwd", args, stream, prepare, R)


def ctr_dot_interaction_bwd(Z: torch.Tensor, dR: torch.Tensor, compute: int = CTR_F32,
                            dZ: Optional[torch.Tensor] = None, stream=None,
                            prepare: bool = False):
    """dZ fp32, or bf16 when ``dZ`` is a bf16 tensor (compute must be CTR_BF16).  Z may be
    bf16 (compute CTR_BF16, dZ bf16)."""
    B, F, d = Z.shape
    if dZ is None:
        dZ = torch.empty_like(Z)
    args = (_ptr(Z), _dtype_code(Z), _ptr(dR), dR.stride(0), B, F, d, compute, _dtype_code(dZ),
            _ptr(dZ))
    return _run("ctr_dot_interaction_bwd", args, stream, prepare, dZ)


def ctr_dot_interaction_self_fwd(Z: torch.Tensor, compute: int = CTR_F32,
                                 R: Optional[torch.Tensor] = None, stream=None,
                                 prepare: bool = False):
    """Pair dots with self-dots (i >= j), P = F(F+1)/2: R = [dense | pairs]."""
    B, F, d = Z.shape
    _require_f32(Z, "ctr_dot_interaction_self_fwd")
    P = F * (F + 1) // 2
    if R is None:
        R = torch.empty((B, d + P), dtype=torch.float32, device=Z.device)
    args = (_ptr(Z), B, F, d, compute, _ptr(R), R.stride(0))
    return _run("ctr_dot_interaction_self_fwd", args, stream, prepare, R)


def ctr_dot_interaction_self_bwd(Z: torch.Tensor, dR: torch.Tensor, compute: int = CTR_F32,
                                 dZ: Optional[torch.Tensor] = None, stream=None,
                                 prepare: bool = False):
    """dZ fp32, or bf16 when ``dZ`` is a bf16 tensor (compute must be CTR_BF16)."""
    B, F, d = Z.shape
    _require_f32(Z, "ctr_dot_interaction_self_bwd")
    if dZ is None:
        dZ = torch.empty_like(Z)
    args = (_ptr(Z), _ptr(dR), dR.stride(0), B, F, d, compute, _dtype_code(dZ), _ptr(dZ))
    return _run("ctr_dot_interaction_self_bwd", args, stream, prepare, dZ)


def ctr_dot_interaction_gram_fwd(Z: torch.Tensor, compute: int = CTR_F32,
                                 R: Optional[torch.Tensor] = None, stream=None,
                                 prepare: bool = False):
    """The whole Gram matrix, P = F^2 row-major after the dense slot: R = [dense | Z Z^T]."""
    B, F, d = Z.shape
    _require_f32(Z, "ctr_dot_interaction_gram_fwd")
    if R is None:
        R = torch.empty((B, d + F * F), dtype=torch.float32, device=Z.device)
    args = (_ptr(Z), B, F, d, compute, _ptr(R), R.stride(0))
    return _run("ctr_dot_interaction_gram_fwd", args, stream, prepare, R)


def ctr_dot_interaction_gram_bwd(Z: torch.Tensor, dR: torch.Tensor, compute: int = CTR_F32,
                                 dZ: Optional[torch.Tensor] = None, stream=None,
                                 prepare: bool = False):
    """dZ_i = sum_j (dG_ij + dG_ji) z_j (+ dense on slot 0); fp32, or bf16 when ``dZ`` is a
    bf16 tensor (compute must be CTR_BF16)."""
    B, F, d = Z.shape
    _require_f32(Z, "ctr_dot_interaction_gram_bwd")
    if dZ is None:
        dZ = torch.empty_like(Z)
    args = (_ptr(Z), _ptr(dR), dR.stride(0), B, F, d, compute, _dtype_code(dZ), _ptr(dZ))
    return _run("ctr_dot_interaction_gram_bwd", args, stream, prepare, dZ)


def ctr_fm_interaction_fwd(Z: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None,
                           prepare: bool = False):
    """Sum of all pair dots per sample by the squared-norm identity: out [B]."""
    B, F, d = Z.shape
    _require_f32(Z, "ctr_fm_interaction_fwd")
    if out is None:
        out = torch.empty((B,), dtype=torch.float32, device=Z.device)
    args = (_ptr(Z), B, F, d, _ptr(out))
    return _run("ctr_fm_interaction_fwd", args, stream, prepare, out)


def ctr_fm_interaction_bwd(Z: torch.Tensor, dout: torch.Tensor,
                           dZ: Optional[torch.Tensor] = None, stream=None,
                           prepare: bool = False):
    B, F, d = Z.shape
    _require_f32(Z, "ctr_fm_interaction_bwd")
    if dZ is None:
        dZ = torch.empty_like(Z)
    args = (_ptr(Z), _ptr(dout), B, F, d, _ptr(dZ))
    return _run("ctr_fm_interaction_bwd", args, stream, prepare, dZ)


def _rows(t: torch.Tensor, name: str):
    """(rows, width, row stride) of a 2-D fp32 view whose rows may be strided."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("%s must be 2-D with contiguous rows" % name)
    return t.shape[0], t.shape[1], t.stride(0)


def dense_bwd_workspace_bytes(M: int, K: int, N: int, bias: bool = True, relu: bool = True,
                              compute: int = CTR_F32) -> int:
    """Workspace of ctr_dense_bwd_sgd for M rows of a K -> N layer (the two-call query)."""
    wsb = ctypes.c_size_t(0)
    b = ctypes.c_void_p(16) if bias else None       # only its presence matters to the query
    _check("ctr_dense_bwd_sgd", load().ctr_dense_bwd_sgd(None, K, M, K, None, b, N,
                                                         int(bool(relu)), None, N, None,
                                                         CTR_F32, N, compute, 0.0, None, K,
                                                         None, ctypes.byref(wsb), None))
    return wsb.value


def ctr_dense_fwd(X: torch.Tensor, W: torch.Tensor, b: Optional[torch.Tensor], relu: bool,
                  compute: int = CTR_F32, Y: Optional[torch.Tensor] = None, stream=None,
                  prepare: bool = False):
    """Y = act(X W^T + b) with X [M, K] (rows may be strided), W [N, K], b [N] or None; Y
    [M, N] (rows may be strided, e.g. Z[:, 0, :])."""
    M, K, xs = _rows(X, "X")
    N = W.shape[0]
    assert W.shape == (N, K) and W.is_contiguous()
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    My, Ny, ys = _rows(Y, "Y")
    assert (My, Ny) == (M, N)
    args = (_ptr(X), xs, M, K, _ptr(W), _ptr(b), N, int(bool(relu)), compute, _ptr(Y), ys)
    return _run("ctr_dense_fwd", args, stream, prepare, Y)


def ctr_dense_bwd_sgd(X: torch.Tensor, W: torch.Tensor, b: Optional[torch.Tensor], relu: bool,
                      Y: Optional[torch.Tensor], dY: torch.Tensor, lr: float,
                      compute: int = CTR_F32, dX: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None,
                      prepare: bool = False):
    """The layer's backward with the SGD step of W and b in place; dX (if given) receives
    dL/dX.  dY: fp32 or bf16 rows (may be strided)."""
    M, K, xs = _rows(X, "X")
    N = W.shape[0]
    _, _, dys = _rows(dY, "dY")
    ys = _rows(Y, "Y")[2] if Y is not None else N
    dxs = _rows(dX, "dX")[2] if dX is not None else K
    if workspace is None:
        workspace = _workspace(dense_bwd_workspace_bytes(M, K, N, b is not None, relu,
                                                         compute), X.device)
    wsb = ctypes.c_size_t(workspace.numel())
    args = (_ptr(X), xs, M, K, _ptr(W), _ptr(b), N, int(bool(relu)), _ptr(Y), ys, _ptr(dY),
            _dtype_code(dY), dys, compute, float(lr), _ptr(dX), dxs, _ptr(workspace),
            ctypes.byref(wsb))
    return _run("ctr_dense_bwd_sgd", args, stream, prepare, dX)


def ctr_logistic_ne(logits: torch.Tensor, labels: torch.Tensor,
                    prob: Optional[torch.Tensor] = None, dlogits: Optional[torch.Tensor] = None,
                    stats: Optional[torch.Tensor] = None, stream=None, prepare: bool = False):
    """Sigmoid, cross-entropy sums and NE of logits [M] (or [M, 1] with any row stride);
    returns stats [3] = [sum ce, sum y, NE] (device).  dlogits, if given, receives the
    gradient of the mean cross-entropy, shaped like logits."""
    M = labels.numel()
    ls = logits.stride(0)
    dls = dlogits.stride(0) if dlogits is not None else 1
    if stats is None:
        stats = torch.empty(3, dtype=torch.float32, device=logits.device)
    args = (_ptr(logits), ls, _ptr(labels), M, _ptr(prob), _ptr(dlogits), dls, _ptr(stats))
    return _run("ctr_logistic_ne", args, stream, prepare, stats)


def ctr_init_tables_hash(table: torch.Tensor, rows: Sequence[int], seed: int,
                         stream=None) -> None:
    lib = load()
    rb = (ctypes.c_int64 * (len(rows) + 1))()
    acc = 0
    for t, r in enumerate(rows):
        rb[t] = acc
        acc += int(r)
    rb[len(rows)] = acc
    _check("ctr_init_tables_hash", lib.ctr_init_tables_hash(
        _ptr(table), _dtype_code(table), table.shape[1], ctypes.cast(rb, ctypes.c_void_p),
        len(rows), ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), _stream(stream)))


def ctr_validate_csr(indices: torch.Tensor, offsets: torch.Tensor, batch: int, num_tables: int,
                     bad_count: torch.Tensor, row_base: Optional[torch.Tensor] = None,
                     total_rows: int = 0, stream=None) -> None:
    lib = load()
    _check("ctr_validate_csr", lib.ctr_validate_csr(
        _ptr(indices), _index_code(indices), indices.numel(), _ptr(offsets), batch, num_tables,
        _ptr(row_base), total_rows, _ptr(bad_count), _stream(stream)))


def ctr_step_run(step: CtrStep, k: int, schedule: int, main_stream=None, side_stream=None,
                 fork_event=None, join_event=None, mark_begin=None, mark_end=None) -> None:
    """Enqueue training step k of ``step`` (a CtrStep) in one native call; the events are
    torch.cuda.Event objects (fork/join required with a side stream)."""
    ms = main_stream if main_stream is not None else torch.cuda.current_stream()

    def ev(e):
        if e is None:
            return None
        if not e.cuda_event:
            e.record(ms)                  # torch creates the HIP event on its first record
        return ctypes.c_void_p(e.cuda_event)

    st = load().ctr_step_run(ctypes.byref(step), k, schedule, ctypes.c_void_p(ms.cuda_stream),
                             None if side_stream is None else ctypes.c_void_p(
                                 side_stream.cuda_stream),
                             ev(fork_event), ev(join_event), ev(mark_begin), ev(mark_end))
    _check("ctr_step_run", st)


def ctr_step_run_deep(step: CtrStep, k: int, main_stream, side_streams, events,
                      mark_begin=None, mark_end=None) -> None:
    """Enqueue step k of the two-deep overlapped schedule; side_streams: two torch streams;
    events: six torch.cuda.Event objects carried between calls."""
    ms = main_stream if main_stream is not None else torch.cuda.current_stream()

    def ev(e):
        if e is None:
            return None
        if not e.cuda_event:
            e.record(ms)                  # torch creates the HIP event on its first record
        return e.cuda_event

    arr = (ctypes.c_void_p * 6)(*[ev(e) for e in events])
    st = load().ctr_step_run_deep(ctypes.byref(step), k, ctypes.c_void_p(ms.cuda_stream),
                                  ctypes.c_void_p(side_streams[0].cuda_stream),
                                  ctypes.c_void_p(side_streams[1].cuda_stream),
                                  ctypes.cast(arr, ctypes.c_void_p),
                                  None if mark_begin is None else ctypes.c_void_p(ev(mark_begin)),
                                  None if mark_end is None else ctypes.c_void_p(ev(mark_end)))
    _check("ctr_step_run_deep", st)


def ctr_step_unique(step: CtrStep, set_index: int, stream=None) -> None:
    _check("ctr_step_unique", load().ctr_step_unique(ctypes.byref(step), set_index,
                                                     _stream(stream)))


# ------------------------------------------------------------------ exported dictionary
def dict_capacity(n: int, load: float = 0.5) -> int:
    """The smallest power-of-two slot count that keeps the table at most `load` full."""
    cap = 2
    while cap * load < n or cap <= n:
        cap *= 2
    return cap


def ctr_dict_build(keys: torch.Tensor, rows: torch.Tensor, hot_slots: Optional[torch.Tensor],
                   capacity: int, slots: Optional[torch.Tensor] = None,
                   status: Optional[torch.Tensor] = None, stream=None):
    """Builds the dictionary's hash table; returns (slots uint8 [capacity*16], status int32[3])."""
    n = keys.numel()
    if slots is None:
        slots = torch.empty(capacity * 16, dtype=torch.uint8, device=keys.device)
    if status is None:
        status = torch.empty(3, dtype=torch.int32, device=keys.device)
    args = (_ptr(keys), _ptr(rows), _ptr(hot_slots), n, _ptr(slots), capacity, _ptr(status))
    _run("ctr_dict_build", args, stream, False)
    return slots, status


def ctr_dict_lookup(ids: torch.Tensor, slots: torch.Tensor, capacity: int,
                    values: Optional[torch.Tensor] = None, stream=None, prepare: bool = False):
    n = ids.numel()
    if values is None:
        values = torch.empty(max(n, 1), dtype=torch.int64, device=ids.device)
    args = (_ptr(ids), n, _ptr(slots), capacity, _ptr(values))
    return _run("ctr_dict_lookup", args, stream, prepare, values)


def _device_view(t: torch.Tensor):
    """Device address of a GPU tensor, or of a pinned host tensor (hipHostGetDevicePointer
    of the HIP runtime already loaded in the process; an error rather than a guess when the
    memory is not device-mapped)."""
    if t.is_cuda:
        return ctypes.c_void_p(t.data_ptr())
    if not t.is_pinned():
        raise ValueError("a host table must be pinned memory")
    global _hip_rt
    if _hip_rt is None:
        path = [ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln][0]
        _hip_rt = ctypes.CDLL(path)
    dptr = ctypes.c_void_p()
    st = _hip_rt.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(t.data_ptr()),
                                         ctypes.c_uint(0))
    if st != 0 or not dptr.value:
        raise RuntimeError("hipHostGetDevicePointer failed (%d)" % st)
    return dptr


_hip_rt = None


def ctr_dict_embbag_fwd(values: torch.Tensor, nnz: int, offsets: torch.Tensor, batch: int,
                        num_tables: int, hot_rows: Optional[torch.Tensor], table: torch.Tensor,
                        out: torch.Tensor, out_stride_b: int, out_stride_t: int, stream=None,
                        prepare: bool = False):
    """Pooled lookup over resolved values; `table` may be a pinned host tensor."""
    num_rows, dim = table.shape
    num_hot = 0 if hot_rows is None else hot_rows.shape[0]
    args = (_ptr(values), nnz, _ptr(offsets), batch, num_tables, _ptr(hot_rows), num_hot,
            _device_view(table), num_rows, _dtype_code(table), dim, _ptr(out), out_stride_b,
            out_stride_t)
    return _run("ctr_dict_embbag_fwd", args, stream, prepare, out)
