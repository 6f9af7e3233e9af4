"""Host-side tests of the C ABI: the library loads, exports every function that
include/ctr.h declares, and rejects bad arguments with the documented status before any
HIP call (so these run without a GPU).  No compute call is made."""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_embedding_lookup_amd import ctr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ctr.h")


def _lib():
    if not os.path.exists(ctr.LIB_PATH):
        from sparse_embedding_lookup_amd import build
        build.build()
    return ctr.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ctr_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_expected_entry_points():
    names = _declared()
    for want in ["ctr_unique_ids", "ctr_gather_rows", "ctr_embbag_fwd", "ctr_embbag_bwd",
                 "ctr_sparse_sgd", "ctr_dot_interaction_fwd", "ctr_dot_interaction_bwd",
                 "ctr_embbag_interaction_fwd"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", ctr.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(ctr_\w+)", out))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    assert set(ctr.EXPORTED) == set(_declared())


FAKE = ctypes.c_void_p(0x10000)       # never dereferenced: every call below fails validation
MISALIGNED = ctypes.c_void_p(0x10004)


def test_status_strings_and_version():
    lib = _lib()
    assert lib.ctr_version() >= 200          # the entry points with layout and type codes
    assert lib.ctr_status_string(0) == b"CTR_OK"
    assert lib.ctr_status_string(3) == b"CTR_ERR_WORKSPACE_TOO_SMALL"


def test_unique_workspace_query_and_bad_args():
    lib = _lib()
    wsb = ctypes.c_size_t(0)
    assert lib.ctr_unique_ids(None, 1, 1000, None, 0, 0, None, 0, 0, 0, None, None, None, None,
                              None, None, 0, None, ctypes.byref(wsb), None) == ctr.CTR_OK
    assert wsb.value >= 1000 * 24
    bad = ctypes.c_size_t(10)
    st = lib.ctr_unique_ids(FAKE, 1, 1000, None, 0, 0, None, 0, 0, 0, FAKE, FAKE, FAKE, None, None,
                            None, 0, FAKE, ctypes.byref(bad), None)
    assert st == ctr.CTR_ERR_WORKSPACE_TOO_SMALL
    big = ctypes.c_size_t(wsb.value)
    st = lib.ctr_unique_ids(FAKE, 1, 1000, None, 0, 0, None, 0, 0, 0, FAKE, FAKE, FAKE, None, None,
                            None, 0, MISALIGNED, ctypes.byref(big), None)
    assert st == ctr.CTR_ERR_UNSUPPORTED and b"aligned" in lib.ctr_last_error_message()
    assert lib.ctr_unique_ids(FAKE, 1, -1, None, 0, 0, None, 0, 0, 0, None, None, None, None, None,
                              None, 0, None, ctypes.byref(wsb), None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_unique_ids(FAKE, 1, 2 ** 31, None, 0, 0, None, 0, 0, 0, None, None, None, None,
                              None, None, 0, None, ctypes.byref(wsb), None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_unique_ids(FAKE, 7, 10, None, 0, 0, None, 0, 0, 0, None, None, None, None, None,
                              None, 0, None, ctypes.byref(wsb), None) == ctr.CTR_ERR_INVALID_ARGUMENT
    # row_base without offsets
    assert lib.ctr_unique_ids(FAKE, 1, 10, None, 4, 2, FAKE, 100, 0, 0, None, None, None, None, None,
                              None, 0, None, ctypes.byref(wsb), None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert b"offsets" in lib.ctr_last_error_message()
    # a negative largest-table hint
    assert lib.ctr_unique_ids(FAKE, 1, 10, FAKE, 4, 2, FAKE, 100, -1, 0, None, None, None, None,
                              None, None, 0, None, ctypes.byref(wsb), None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT


def test_embbag_fwd_bad_args():
    lib = _lib()
    ok = dict(table=FAKE, dtype=0, rows=100, dim=16, rb=None, T=1, idx=FAKE, it=1, nnz=10,
              off=FAKE, B=10, out=FAKE, ot=0, sb=16, st=0, ws=FAKE, wsb=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        wsb = ctypes.c_size_t(a["wsb"])
        return lib.ctr_embbag_fwd(a["table"], a["dtype"], a["rows"], a["dim"], a["rb"], a["T"],
                                  a["idx"], a["it"], a["nnz"], a["off"], a["B"], a["out"],
                                  a["ot"], a["sb"], a["st"], a["ws"], ctypes.byref(wsb), None)

    # the workspace query needs nnz and dim only: 256 bytes up to 4096 occurrences, then the
    # long bags' chunk partials
    q = ctypes.c_size_t(0)
    assert lib.ctr_embbag_fwd(None, 0, 0, 16, None, 1, None, 1, 4096, None, 0, None, 0, 0, 0,
                              None, ctypes.byref(q), None) == ctr.CTR_OK and q.value == 256
    assert lib.ctr_embbag_fwd(None, 0, 0, 16, None, 1, None, 1, 1 << 20, None, 0, None, 0, 0, 0,
                              None, ctypes.byref(q), None) == ctr.CTR_OK
    assert q.value == 256 + 256 * 8 + 256 * 2 * 16 * 4
    assert ctr.embbag_fwd_workspace_bytes(1 << 20, 16) == q.value
    assert call(wsb=q.value - 1, nnz=1 << 20) == ctr.CTR_ERR_WORKSPACE_TOO_SMALL
    assert call(ws=MISALIGNED) == ctr.CTR_ERR_UNSUPPORTED

    assert call(table=None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(dtype=5) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(dim=6) == ctr.CTR_ERR_UNSUPPORTED              # not a 16-byte multiple (fp32)
    assert call(dtype=1, dim=12) == ctr.CTR_ERR_UNSUPPORTED    # bf16 needs multiples of 8
    assert call(dtype=ctr.CTR_F16, dim=12) == ctr.CTR_ERR_UNSUPPORTED   # so does fp16
    assert call(dtype=3) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(table=MISALIGNED) == ctr.CTR_ERR_UNSUPPORTED
    assert call(out=MISALIGNED) == ctr.CTR_ERR_UNSUPPORTED
    assert call(sb=18) == ctr.CTR_ERR_UNSUPPORTED
    # bf16 pooled vectors: stores of up to 8 values, so strides in multiples of 8
    assert call(ot=ctr.CTR_BF16, sb=20) == ctr.CTR_ERR_UNSUPPORTED
    assert call(ot=7) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert b"out_dtype" in lib.ctr_last_error_message()
    assert call(it=3) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(nnz=-1) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(off=None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(T=0) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(dim=2048) == ctr.CTR_ERR_UNSUPPORTED


def test_embbag_interaction_fwd_bad_args():
    lib = _lib()
    # a valid call: 4 tables (F = 5) of d = 16 fp32, P = 10, so r_stride >= 26
    ok = dict(table=FAKE, dtype=0, rows=100, dim=16, rb=None, T=4, idx=FAKE, it=1, nnz=10,
              off=FAKE, B=10, Z=FAKE, c=0, R=FAKE, rs=26)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.ctr_embbag_interaction_fwd(a["table"], a["dtype"], a["rows"], a["dim"],
                                              a["rb"], a["T"], a["idx"], a["it"], a["nnz"],
                                              a["off"], a["B"], a["Z"], a["c"], a["R"], a["rs"],
                                              None)

    assert call(table=None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(dtype=5) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(dim=6) == ctr.CTR_ERR_UNSUPPORTED              # not a 16-byte multiple
    assert call(dtype=ctr.CTR_F16) == ctr.CTR_ERR_UNSUPPORTED  # fp16 tables: separate calls
    assert b"CTR_F16" in lib.ctr_last_error_message()
    assert call(it=3) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(T=0) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(nnz=-1) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(c=7) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(off=None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(Z=None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(R=None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(idx=None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert call(rs=25) == ctr.CTR_ERR_INVALID_ARGUMENT        # < dim + P
    assert call(Z=MISALIGNED) == ctr.CTR_ERR_UNSUPPORTED
    assert call(table=MISALIGNED) == ctr.CTR_ERR_UNSUPPORTED
    assert call(dim=48, rs=58) == ctr.CTR_ERR_UNSUPPORTED             # 12 vectors: not a power of two
    assert call(dim=256, rs=266) == ctr.CTR_ERR_UNSUPPORTED            # 64 vectors: above 32
    assert call(T=300, rs=16 + 301 * 300 // 2) == ctr.CTR_ERR_UNSUPPORTED   # > 256 tables
    assert call(c=1, dim=8, dtype=1) == ctr.CTR_ERR_UNSUPPORTED  # bf16 compute: dim >= 16
    assert call(c=1, T=128, rs=16 + 129 * 128 // 2) == ctr.CTR_ERR_UNSUPPORTED   # F > 128
    # an fp32 copy of one sample above 46 KiB: F = 101, d = 128 -> 52 KB
    assert call(dim=128, T=100, rs=128 + 101 * 50) == ctr.CTR_ERR_UNSUPPORTED
    assert b"fused shape" in lib.ctr_last_error_message()
    # batch 0 is a no-op that launches nothing
    assert call(B=0, nnz=0, idx=None, off=None, Z=None, R=None) == ctr.CTR_OK


def test_embbag_bwd_workspace_and_bad_args():
    lib = _lib()
    wsb = ctypes.c_size_t(0)
    assert lib.ctr_embbag_bwd(None, 64, 0, None, 10, 1, 64, 1000, None, None, None, None, None,
                              None, ctypes.byref(wsb), None) == ctr.CTR_OK
    assert wsb.value >= 1000 * 12
    assert lib.ctr_embbag_bwd(None, 64, 0, None, 10, 1, 6, 1000, None, None, None, None, None,
                              None, ctypes.byref(wsb), None) == ctr.CTR_ERR_UNSUPPORTED
    small = ctypes.c_size_t(16)
    assert lib.ctr_embbag_bwd(FAKE, 64, 0, FAKE, 10, 1, 64, 1000, FAKE, FAKE, None, FAKE, FAKE,
                              FAKE, ctypes.byref(small), None) == ctr.CTR_ERR_WORKSPACE_TOO_SMALL
    big = ctypes.c_size_t(wsb.value)
    assert lib.ctr_embbag_bwd(MISALIGNED, 64, 0, FAKE, 10, 1, 64, 1000, FAKE, FAKE, None, FAKE,
                              FAKE, FAKE, ctypes.byref(big), None) == ctr.CTR_ERR_UNSUPPORTED
    # neither sorted_src nor (perm, inverse)
    assert lib.ctr_embbag_bwd(FAKE, 64, 0, FAKE, 10, 1, 64, 1000, None, FAKE, None, FAKE, FAKE,
                              FAKE, ctypes.byref(big), None) == ctr.CTR_ERR_INVALID_ARGUMENT


def test_interaction_bad_args():
    lib = _lib()
    f = lambda Z, *a, zt=0: lib.ctr_dot_interaction_fwd(Z, zt, *a)
    assert f(FAKE, 10, 1, 16, 0, FAKE, 100, None) == ctr.CTR_ERR_INVALID_ARGUMENT    # F < 2
    assert f(FAKE, 10, 5, 16, 0, FAKE, 20, None) == ctr.CTR_ERR_INVALID_ARGUMENT     # stride
    assert f(FAKE, 10, 5, 16, 9, FAKE, 26, None) == ctr.CTR_ERR_INVALID_ARGUMENT     # compute
    assert f(FAKE, 10, 5, 24, 1, FAKE, 40, None) == ctr.CTR_ERR_UNSUPPORTED          # bf16 dim
    assert f(FAKE, 10, 200, 128, 1, FAKE, 30000, None) == ctr.CTR_ERR_UNSUPPORTED    # bf16 F
    assert f(MISALIGNED, 10, 5, 16, 1, FAKE, 26, None) == ctr.CTR_ERR_UNSUPPORTED
    # a bf16 Z: only for the matrix-core interaction; an unknown Z type
    assert f(FAKE, 10, 5, 16, 0, FAKE, 26, None, zt=ctr.CTR_BF16) == ctr.CTR_ERR_UNSUPPORTED
    assert f(FAKE, 10, 5, 16, 1, FAKE, 26, None, zt=5) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert b"z_dtype" in lib.ctr_last_error_message()
    b = lambda Z, *a, zt=0: lib.ctr_dot_interaction_bwd(Z, zt, *a)
    assert b(FAKE, None, 26, 10, 5, 16, 0, 0, FAKE, None) == ctr.CTR_ERR_INVALID_ARGUMENT  # dR NULL
    # dZ type: an unknown code, and bf16 storage without bf16 compute
    assert b(FAKE, FAKE, 26, 10, 5, 16, 1, 7, FAKE, None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert b"dz_dtype" in lib.ctr_last_error_message()
    assert b(FAKE, FAKE, 26, 10, 5, 16, 0, 1, FAKE, None) == ctr.CTR_ERR_UNSUPPORTED
    # the matrix-core backward stores dZ as 8- and 16-byte vectors
    assert b(FAKE, FAKE, 26, 10, 5, 16, 1, 1, MISALIGNED, None) == ctr.CTR_ERR_UNSUPPORTED
    assert b"dZ is not 16-byte aligned" in lib.ctr_last_error_message()
    assert b(FAKE, FAKE, 26, 10, 5, 16, 1, 0, MISALIGNED, None) == ctr.CTR_ERR_UNSUPPORTED
    # a bf16 Z takes a bf16 dZ, and bf16 compute
    assert b(FAKE, FAKE, 26, 10, 5, 16, 1, 0, FAKE, None, zt=ctr.CTR_BF16) == \
        ctr.CTR_ERR_UNSUPPORTED
    assert b(FAKE, FAKE, 26, 10, 5, 16, 0, 0, FAKE, None, zt=ctr.CTR_BF16) == \
        ctr.CTR_ERR_UNSUPPORTED


def test_sgd_gather_init_validate_bad_args():
    lib = _lib()
    s0 = ctypes.c_uint64(0)
    assert lib.ctr_sparse_sgd(FAKE, 0, 100, 16, FAKE, FAKE, 10, FAKE,
                              ctypes.c_float(float("nan")), 0, s0, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_sparse_sgd(FAKE, 0, 100, 16, FAKE, FAKE, 10, MISALIGNED,
                              ctypes.c_float(0.01), 0, s0, None) == ctr.CTR_ERR_UNSUPPORTED
    assert lib.ctr_gather_rows(FAKE, 0, 100, 16, None, FAKE, 10, FAKE, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    rb = (ctypes.c_int64 * 3)(0, 10, 5)                    # decreasing
    assert lib.ctr_init_tables_hash(FAKE, 0, 16, ctypes.cast(rb, ctypes.c_void_p), 2,
                                    ctypes.c_uint64(1), None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_validate_csr(FAKE, 1, 10, None, 10, 1, None, 100, FAKE, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT


def test_rounding_argument_bad_args():
    lib = _lib()
    s0 = ctypes.c_uint64(7)
    SR = ctr.CTR_ROUND_STOCHASTIC
    # fp32 tables have no stochastic rounding; an unknown rounding code
    st = lib.ctr_sparse_sgd(FAKE, ctr.CTR_F32, 100, 16, FAKE, FAKE, 10, FAKE,
                            ctypes.c_float(0.01), SR, s0, None)
    assert st == ctr.CTR_ERR_UNSUPPORTED and b"BF16" in lib.ctr_last_error_message()
    assert lib.ctr_sparse_sgd(FAKE, ctr.CTR_BF16, 100, 16, FAKE, FAKE, 10, FAKE,
                              ctypes.c_float(float("inf")), SR, s0, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_sparse_sgd(FAKE, ctr.CTR_BF16, 100, 16, FAKE, FAKE, 10, FAKE,
                              ctypes.c_float(0.01), 5, s0, None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert b"rounding" in lib.ctr_last_error_message()
    # fp16 tables take both roundings (the query of the fused backward answers)
    wsb = ctypes.c_size_t(0)
    assert lib.ctr_embbag_bwd_sgd(None, ctr.CTR_F32, 64, 0, None, 10, 1, 100, None, 0, None, FAKE,
                                  ctr.CTR_F16, 1000, 16, None, ctypes.c_float(0.01), SR, s0,
                                  None, None, ctypes.byref(wsb), None) == ctr.CTR_OK
    assert wsb.value > 0
    wsb = ctypes.c_size_t(0)
    bwd = lib.ctr_embbag_bwd_sgd
    st = bwd(FAKE, ctr.CTR_F32, 64, 0, FAKE, 10, 1, 100, FAKE, 0, FAKE, FAKE, ctr.CTR_F32, 1000, 16,
             FAKE, ctypes.c_float(0.01), SR, s0, None, None, ctypes.byref(wsb), None)
    assert st == ctr.CTR_ERR_UNSUPPORTED
    assert bwd(FAKE, ctr.CTR_F32, 64, 0, FAKE, 10, 1, 100, FAKE, 0, FAKE, FAKE, ctr.CTR_BF16, 1000,
               16, FAKE, ctypes.c_float(0.01), 9, s0, None, None, ctypes.byref(wsb), None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert bwd(FAKE, 4, 64, 0, FAKE, 10, 1, 100, FAKE, 0, FAKE, FAKE, ctr.CTR_BF16, 1000, 16, FAKE,
               ctypes.c_float(0.01), 0, s0, None, None, ctypes.byref(wsb), None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert b"grad_dtype" in lib.ctr_last_error_message()
    assert bwd(None, ctr.CTR_F32, 64, 0, None, 10, 1, 100, None, 0, None, FAKE, ctr.CTR_BF16, 1000,
               16, None, ctypes.c_float(0.01), SR, s0, None, None, ctypes.byref(wsb), None) == \
        ctr.CTR_OK
    assert wsb.value > 0                          # the workspace query of ctr_embbag_bwd


def test_interaction_variant_bad_args():
    lib = _lib()
    f = lib.ctr_dot_interaction_self_fwd
    # F = 5, dim = 16: the self-dot set needs dim + 15 columns, the strict one dim + 10
    assert f(FAKE, 10, 5, 16, ctr.CTR_F32, FAKE, 16 + 10, None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert b"stride" in lib.ctr_last_error_message()
    assert f(FAKE, 10, 0, 16, ctr.CTR_F32, FAKE, 100, None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert f(FAKE, 10, 5, 24, ctr.CTR_BF16, FAKE, 100, None) == ctr.CTR_ERR_UNSUPPORTED
    b = lib.ctr_dot_interaction_self_bwd
    assert b(FAKE, None, 31, 10, 5, 16, ctr.CTR_F32, ctr.CTR_F32, FAKE, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    # the Gram matrix: F^2 entries after the dense slot, F >= 1
    g = lib.ctr_dot_interaction_gram_fwd
    assert g(FAKE, 10, 5, 16, ctr.CTR_F32, FAKE, 16 + 24, None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert g(FAKE, 10, 0, 16, ctr.CTR_F32, FAKE, 100, None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert g(FAKE, 10, 5000, 16, ctr.CTR_F32, FAKE, 1 << 26, None) == ctr.CTR_ERR_UNSUPPORTED
    assert g(None, 0, 5, 16, ctr.CTR_F32, None, 16 + 25, None) == ctr.CTR_OK      # empty batch
    gb = lib.ctr_dot_interaction_gram_bwd
    assert gb(FAKE, None, 41, 10, 5, 16, ctr.CTR_F32, ctr.CTR_F32, FAKE, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert gb(FAKE, FAKE, 41, 10, 5, 16, ctr.CTR_F32, ctr.CTR_BF16, FAKE, None) == \
        ctr.CTR_ERR_UNSUPPORTED
    assert lib.ctr_fm_interaction_fwd(FAKE, 10, 0, 16, FAKE, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_fm_interaction_bwd(FAKE, None, 10, 3, 16, FAKE, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_fm_interaction_fwd(None, 0, 3, 16, None, None) == ctr.CTR_OK   # empty batch


def test_dictionary_bad_args():
    lib = _lib()
    st32 = FAKE
    # capacity must be a power of two above n
    assert lib.ctr_dict_build(FAKE, FAKE, None, 10, FAKE, 12, st32, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_dict_build(FAKE, FAKE, None, 16, FAKE, 16, st32, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert b"capacity" in lib.ctr_last_error_message()
    assert lib.ctr_dict_build(FAKE, FAKE, None, 10, MISALIGNED, 16, st32, None) == \
        ctr.CTR_ERR_UNSUPPORTED
    assert lib.ctr_dict_lookup(FAKE, 10, FAKE, 100, FAKE, None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_dict_lookup(FAKE, 10, None, 64, FAKE, None) == ctr.CTR_ERR_INVALID_ARGUMENT
    p = lib.ctr_dict_embbag_fwd
    # an empty dictionary table, a cache count without a cache, misaligned output
    assert p(FAKE, 10, FAKE, 10, 1, None, 0, FAKE, 0, ctr.CTR_F32, 32, FAKE, 32, 0, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert p(FAKE, 10, FAKE, 10, 1, None, 5, FAKE, 100, ctr.CTR_F32, 32, FAKE, 32, 0, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert p(FAKE, 10, FAKE, 10, 1, None, 0, FAKE, 100, ctr.CTR_F32, 32, MISALIGNED, 32, 0,
             None) == ctr.CTR_ERR_UNSUPPORTED


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(ctr, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(ctr, "_lib", None)
    with pytest.raises(RuntimeError):
        ctr.load()


def test_step_struct_layout_matches_header(tmp_path):
    """The binding's CtrStep has the size and field offsets of ctr_step_t (checked with the
    host C compiler against include/ctr.h)."""
    fields = [f for f, _ in ctr.CtrStep._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "%s"\nint main(void){'
                   'printf("size %%zu\\n", sizeof(ctr_step_t));%s return 0;}\n'
                   % (HEADER, "".join('printf("%s %%zu\\n", offsetof(ctr_step_t, %s));' % (f, f)
                                      for f in fields)))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-o", str(exe), str(src)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True,
                                                       text=True, check=True).stdout.splitlines())
    assert int(got["size"]) == ctypes.sizeof(ctr.CtrStep)
    for f in fields:
        assert getattr(ctr.CtrStep, f).offset == int(got[f]), f


def test_step_run_bad_args():
    lib = _lib()
    d = ctr.CtrStep()
    assert lib.ctr_step_run(None, 0, 0, None, None, None, None, None, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    d.kind = 7
    assert lib.ctr_step_run(ctypes.byref(d), 0, 0, None, None, None, None, None, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    d.kind = ctr.CTR_STEP_POOLED_INTERACTION
    # pipelined without a side stream; side stream without events; negative step; bad schedule
    assert lib.ctr_step_run(ctypes.byref(d), 0, ctr.CTR_SCHEDULE_PIPELINED, None, None, None,
                            None, None, None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_step_run(ctypes.byref(d), 0, 0, None, FAKE, None, None, None, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_step_run(ctypes.byref(d), -1, 0, None, None, None, None, None, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_step_run(ctypes.byref(d), 0, 5, None, None, None, None, None, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_step_unique(ctypes.byref(d), 3, None) == ctr.CTR_ERR_INVALID_ARGUMENT
    # the two-deep schedule: two side streams, six events and a second unique workspace
    ev6 = (ctypes.c_void_p * 6)(*([0x10000] * 6))
    assert lib.ctr_step_run_deep(ctypes.byref(d), 0, None, FAKE, None, ctypes.cast(ev6, ctypes.c_void_p),
                                 None, None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_step_run_deep(ctypes.byref(d), 0, None, FAKE, FAKE, None, None, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_step_run_deep(ctypes.byref(d), 0, None, FAKE, FAKE,
                                 ctypes.cast(ev6, ctypes.c_void_p), None, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert b"workspace" in lib.ctr_last_error_message()



def test_dense_and_head_bad_args():
    lib = _lib()
    fwd = dict(X=FAKE, xs=13, M=10, K=13, W=FAKE, b=None, N=4, relu=1, c=0, Y=FAKE, ys=4)

    def f(**kw):
        a = dict(fwd, **kw)
        return lib.ctr_dense_fwd(a["X"], a["xs"], a["M"], a["K"], a["W"], a["b"], a["N"],
                                 a["relu"], a["c"], a["Y"], a["ys"], None)

    assert f(K=0) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert f(N=70000) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert f(c=7) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert f(xs=12) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert f(ys=3) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert f(W=None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert f(M=-1) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert f(M=1 << 22, N=1024, ys=1024) == ctr.CTR_ERR_INVALID_ARGUMENT       # M * N >= 2^31
    # backward: workspace query, then a too-small and a misaligned workspace
    wsb = ctypes.c_size_t(0)
    assert lib.ctr_dense_bwd_sgd(None, 13, 10, 13, None, None, 4, 1, None, 4, None, 0, 4, 0,
                                 0.1, None, 13, None, ctypes.byref(wsb), None) == ctr.CTR_OK
    assert wsb.value >= 10 * 4 * 4                                    # dA of a ReLU layer
    assert wsb.value == ctr.dense_bwd_workspace_bytes(10, 13, 4, bias=False)
    # zero rows: a valid query (no tiles to split)
    assert ctr.dense_bwd_workspace_bytes(0, 13, 4) >= 16
    assert ctr.dense_bwd_workspace_bytes(0, 2048, 2048, compute=ctr.CTR_BF16) >= 16
    # bf16 compute keeps dA in bf16; a linear layer needs no dA
    assert ctr.dense_bwd_workspace_bytes(1000, 13, 64, compute=ctr.CTR_BF16) < \
        ctr.dense_bwd_workspace_bytes(1000, 13, 64)
    assert ctr.dense_bwd_workspace_bytes(1000, 13, 64, relu=False) < 1000 * 64 * 2
    # a split reduction (few output tiles, many rows) needs its partials
    assert ctr.dense_bwd_workspace_bytes(100000, 64, 64, relu=False) >= 2 * 64 * 65 * 4

    def bw(ws, size, **kw):
        a = dict(dt=0, dys=4, relu=1, Y=FAKE, dX=None, dxs=13)
        a.update(kw)
        s = ctypes.c_size_t(size)
        return lib.ctr_dense_bwd_sgd(FAKE, 13, 10, 13, FAKE, None, 4, a["relu"], a["Y"], 4, FAKE,
                                     a["dt"], a["dys"], 0, 0.1, a["dX"], a["dxs"], ws,
                                     ctypes.byref(s), None)

    assert bw(FAKE, 8) == ctr.CTR_ERR_WORKSPACE_TOO_SMALL
    assert bw(MISALIGNED, wsb.value) == ctr.CTR_ERR_UNSUPPORTED
    assert bw(FAKE, wsb.value, dt=3) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert bw(FAKE, wsb.value, dys=2) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert bw(FAKE, wsb.value, dX=FAKE, dxs=5) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert bw(FAKE, wsb.value, Y=None) == ctr.CTR_ERR_INVALID_ARGUMENT     # ReLU needs Y
    assert lib.ctr_dense_bwd_sgd(FAKE, 13, 10, 13, FAKE, None, 4, 1, FAKE, 4, FAKE, 0, 4, 0, 0.1,
                                 None, 13, FAKE, None, None) == ctr.CTR_ERR_INVALID_ARGUMENT
    # head
    assert lib.ctr_logistic_ne(FAKE, 1, FAKE, 0, None, None, 1, FAKE, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_logistic_ne(FAKE, 1, None, 5, None, None, 1, FAKE, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_logistic_ne(FAKE, 0, FAKE, 5, None, None, 1, FAKE, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT
    assert lib.ctr_logistic_ne(FAKE, 1, FAKE, 5, None, None, 1, None, None) == \
        ctr.CTR_ERR_INVALID_ARGUMENT


def test_row_entry_layout_rejections():
    """CTR_SRC_ROWS (8-byte (row, bag) entries): an unknown layout, keys that need more than
    31 bits, 8-byte misalignment, and a backward that would need u (row gradients, no table)
    are rejected before any launch."""
    lib = _lib()
    wsb = ctypes.c_size_t(0)
    assert lib.ctr_unique_ids(None, 1, 1000, None, 0, 0, None, 0, 0, 0, None, None, None, None,
                              None, None, 0, None, ctypes.byref(wsb), None) == ctr.CTR_OK
    big = ctypes.c_size_t(wsb.value)
    uq = lambda *a: lib.ctr_unique_ids(*a, FAKE, ctypes.byref(big), None)
    # (ids, id_type, n, offsets, batch, T, row_base, total_rows, max_rows, modulus, uniq, inv,
    #  num_unique, perm, seg, sorted_src, src_layout)
    assert uq(FAKE, 1, 1000, None, 0, 0, None, 0, 0, 0, FAKE, FAKE, FAKE, None, None, FAKE,
              5) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert b"src_layout" in lib.ctr_last_error_message()
    # raw int64 keys (no row_base, no modulus) do not fit the 32-bit key of a row entry
    assert uq(FAKE, 1, 1000, None, 0, 0, None, 0, 0, 0, FAKE, FAKE, FAKE, None, None, FAKE,
              ctr.CTR_SRC_ROWS) == ctr.CTR_ERR_UNSUPPORTED
    assert uq(FAKE, 1, 1000, None, 0, 0, None, 0, 0, (1 << 31) + 1, FAKE, FAKE, FAKE, None,
              None, FAKE, ctr.CTR_SRC_ROWS) == ctr.CTR_ERR_UNSUPPORTED
    assert uq(FAKE, 1, 1000, FAKE, 4, 2, FAKE, 1 << 31, 0, 0, FAKE, FAKE, FAKE, None, None,
              FAKE, ctr.CTR_SRC_ROWS) == ctr.CTR_ERR_UNSUPPORTED
    assert uq(FAKE, 1, 1000, None, 0, 0, None, 0, 0, 1000, FAKE, FAKE, FAKE, None, None,
              MISALIGNED, ctr.CTR_SRC_ROWS) == ctr.CTR_ERR_UNSUPPORTED
    assert b"8-byte" in lib.ctr_last_error_message()
    # the backward: (grad, grad_dtype, sb, st, offsets, batch, T, nnz, sorted_src, src_layout,
    #  num_unique, table, dtype, total_rows, dim, uniq, lr, rounding, seed, row_grads, ws, wsb)
    lr, s0 = ctypes.c_float(0.01), ctypes.c_uint64(0)
    wsb = ctypes.c_size_t(0)
    assert lib.ctr_embbag_bwd_sgd(None, ctr.CTR_F32, 64, 0, None, 10, 1, 100, None,
                                  ctr.CTR_SRC_ROWS, None, FAKE, ctr.CTR_F32, 1000, 16, None, lr,
                                  0, s0, None, None, ctypes.byref(wsb), None) == ctr.CTR_OK
    big = ctypes.c_size_t(wsb.value)
    bwd = lambda *a: lib.ctr_embbag_bwd_sgd(*a, FAKE, ctypes.byref(big), None)
    assert bwd(FAKE, ctr.CTR_F32, 64, 0, FAKE, 10, 1, 100, FAKE, 3, FAKE, FAKE, ctr.CTR_F32,
               1000, 16, None, lr, 0, s0, None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert b"src_layout" in lib.ctr_last_error_message()
    # row gradients are indexed by u, which row entries do not carry
    assert bwd(FAKE, ctr.CTR_F32, 64, 0, FAKE, 10, 1, 100, FAKE, ctr.CTR_SRC_ROWS, FAKE, FAKE,
               ctr.CTR_F32, 1000, 16, None, lr, 0, s0, FAKE) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert b"row_grads" in lib.ctr_last_error_message()
    assert bwd(FAKE, ctr.CTR_F32, 64, 0, FAKE, 10, 1, 100, FAKE, ctr.CTR_SRC_ROWS, FAKE, None,
               ctr.CTR_F32, 1000, 16, None, lr, 0, s0, FAKE) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert bwd(FAKE, ctr.CTR_F32, 64, 0, FAKE, 10, 1, 100, MISALIGNED, ctr.CTR_SRC_ROWS, FAKE,
               FAKE, ctr.CTR_F32, 1000, 16, None, lr, 0, s0, None) == ctr.CTR_ERR_UNSUPPORTED
    assert b"8-byte" in lib.ctr_last_error_message()
    # the quadruple layout still needs uniq with a table
    assert bwd(FAKE, ctr.CTR_F32, 64, 0, FAKE, 10, 1, 100, FAKE, ctr.CTR_SRC_FULL, FAKE, FAKE,
               ctr.CTR_F32, 1000, 16, None, lr, 0, s0, None) == ctr.CTR_ERR_INVALID_ARGUMENT
    assert b"uniq" in lib.ctr_last_error_message()


def test_noalloc_backward_limits_and_rejections():
    """The backward that allocates nothing: a fixed per-GPU scratch (64 MiB), a size query,
    and batches beyond it rejected on the host before any launch (fake device pointers)."""
    lib = _lib()
    assert lib.ctr_noalloc_scratch_capacity() == 64 << 20
    small = lib.ctr_embbag_bwd_noalloc_scratch_bytes(327680, 64)
    assert 0 < small < 64 << 20
    assert lib.ctr_embbag_bwd_noalloc_scratch_bytes(67_000_000, 128) > 64 << 20
    assert lib.ctr_embbag_bwd_noalloc_scratch_bytes(-1, 64) == ctypes.c_size_t(-1).value
    args = (FAKE, 1, 65 * 128, 128, FAKE, 32768, 64, 67_000_000, FAKE, 0, FAKE, FAKE, 1,
            256_000_000, 128, FAKE, ctypes.c_float(0.01), 0, ctypes.c_uint64(0), None, None)
    assert lib.ctr_embbag_bwd_sgd_noalloc(*args) == 2          # CTR_ERR_UNSUPPORTED
    assert b"scratch" in lib.ctr_last_error_message()
    bad = list(args)
    bad[1] = 7                                                 # unknown gradient dtype
    assert lib.ctr_embbag_bwd_sgd_noalloc(*bad) == 1
    bad = list(args)
    bad[17] = 9                                                # unknown rounding
    assert lib.ctr_embbag_bwd_sgd_noalloc(*bad) == 1


def test_binding_workspace_queries():
    """The binding's two-call size queries run on the host (no device memory touched)."""
    _lib()
    assert ctr.unique_workspace_bytes(1000) >= 1000 * 16
    assert ctr.unique_workspace_bytes(2_000_000) > ctr.unique_workspace_bytes(1000)
    assert ctr.embbag_bwd_workspace_bytes(1000, 64) > 0
