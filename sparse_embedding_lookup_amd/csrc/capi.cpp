// capi.cpp -- the C ABI of libctr: host-side argument checks, workspace sizing, launches.
// Every check runs before the first HIP call, so a bad argument never touches the device.
#include <stdarg.h>
#include <stdio.h>

#include <cmath>

#include "../../include/ctr.h"
#include "ctr_internal.h"

namespace {

thread_local char g_msg[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

int32_t hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return CTR_OK;
  return fail(CTR_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// Alignment mask of sorted_src: 16-byte quadruples, or 8-byte row entries.
uintptr_t src_align(int32_t layout) { return layout == CTR_SRC_ROWS ? 7u : 15u; }

constexpr int64_t kMaxElems = 2147483647;  // int32 positions and indices

int bitlen(uint64_t x) {
  int b = 0;
  while (x) {
    ++b;
    x >>= 1;
  }
  return b;
}

// The kernels' element-type codes are the table dtype codes.
static_assert(ctr::kEltF32 == CTR_F32 && ctr::kEltBF16 == CTR_BF16 && ctr::kEltF16 == CTR_F16,
              "table element codes");

int32_t check_table(const void* table, int32_t dtype, int64_t total_rows, int32_t dim) {
  if (!table) return fail(CTR_ERR_INVALID_ARGUMENT, "table is NULL");
  if (dtype != CTR_F32 && dtype != CTR_BF16 && dtype != CTR_F16)
    return fail(CTR_ERR_INVALID_ARGUMENT, "dtype %d is not CTR_F32, CTR_BF16 or CTR_F16", dtype);
  if (total_rows < 0) return fail(CTR_ERR_INVALID_ARGUMENT, "total_rows < 0");
  if (dim <= 0) return fail(CTR_ERR_INVALID_ARGUMENT, "dim must be positive");
  const int e = dtype != CTR_F32 ? 8 : 4;
  if (dim % e != 0)
    return fail(CTR_ERR_UNSUPPORTED, "dim %d is not a multiple of the 16-byte vector (%d)", dim, e);
  if (dim / e > 256) return fail(CTR_ERR_UNSUPPORTED, "dim %d above the 4 KiB row limit", dim);
  if (!aligned16(table)) return fail(CTR_ERR_UNSUPPORTED, "table is not 16-byte aligned");
  return CTR_OK;
}

}  // namespace

namespace ctr {
int32_t set_error(int32_t code, const char* msg) { return fail(code, "%s", msg); }

hipError_t record_mark(void* ev, hipStream_t s) {
  if (!ev) return hipSuccess;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &cs);
  if (e != hipSuccess) return e;
  if (cs != hipStreamCaptureStatusActive) return hipEventRecord(static_cast<hipEvent_t>(ev), s);
  hipStreamCaptureStatus st;
  unsigned long long id;
  hipGraph_t g;
  const hipGraphNode_t* deps;
  size_t ndeps;
  hipGraphNode_t node;
  e = hipStreamGetCaptureInfo_v2(s, &st, &id, &g, &deps, &ndeps);
  if (e == hipSuccess)
    e = hipGraphAddEventRecordNode(&node, g, deps, ndeps, static_cast<hipEvent_t>(ev));
  if (e == hipSuccess)
    e = hipStreamUpdateCaptureDependencies(s, &node, 1, hipStreamSetCaptureDependencies);
  return e;
}
}  // namespace ctr

extern "C" {

// 0.2.0: sorted_src layouts (src_layout), bf16 pooled vectors (out_dtype) and bf16 Z (z_dtype)
int32_t ctr_version(void) { return 200; }

const char* ctr_status_string(int32_t status) {
  switch (status) {
    case CTR_OK: return "CTR_OK";
    case CTR_ERR_INVALID_ARGUMENT: return "CTR_ERR_INVALID_ARGUMENT";
    case CTR_ERR_UNSUPPORTED: return "CTR_ERR_UNSUPPORTED";
    case CTR_ERR_WORKSPACE_TOO_SMALL: return "CTR_ERR_WORKSPACE_TOO_SMALL";
    case CTR_ERR_HIP: return "CTR_ERR_HIP";
    default: return "CTR_ERR_UNKNOWN";
  }
}

const char* ctr_last_error_message(void) { return g_msg; }

int32_t ctr_unique_ids(const void* ids, int32_t id_type, int64_t n, const int64_t* offsets,
                       int64_t batch, int32_t num_tables, const int64_t* row_base,
                       int64_t total_rows, int64_t max_table_rows, int64_t key_modulus,
                       int64_t* uniq,
                       int32_t* inverse, int32_t* num_unique, int32_t* perm,
                       int32_t* seg_offsets, int32_t* sorted_src, int32_t src_layout,
                       void* workspace, size_t* workspace_bytes, void* stream) {
  g_msg[0] = 0;
  if (!workspace_bytes) return fail(CTR_ERR_INVALID_ARGUMENT, "workspace_bytes is NULL");
  if (src_layout != CTR_SRC_FULL && src_layout != CTR_SRC_ROWS)
    return fail(CTR_ERR_INVALID_ARGUMENT, "src_layout %d is not CTR_SRC_FULL or CTR_SRC_ROWS",
                src_layout);
  // row entries hold the key in 32 bits: keys below 2^31 (table rows, or a modulus)
  if (src_layout == CTR_SRC_ROWS && !(row_base ? total_rows <= kMaxElems
                                               : (key_modulus > 0 && key_modulus <= kMaxElems + 1)))
    return fail(CTR_ERR_UNSUPPORTED,
                "CTR_SRC_ROWS needs keys below 2^31 (total_rows with row_base, or key_modulus)");
  if (n < 0 || n > kMaxElems) return fail(CTR_ERR_INVALID_ARGUMENT, "n=%lld out of [0, 2^31)", (long long)n);
  if (id_type != CTR_I32 && id_type != CTR_I64)
    return fail(CTR_ERR_INVALID_ARGUMENT, "id_type %d is not CTR_I32 or CTR_I64", id_type);
  if (key_modulus < 0) return fail(CTR_ERR_INVALID_ARGUMENT, "key_modulus < 0");
  if (row_base) {
    if (!offsets) return fail(CTR_ERR_INVALID_ARGUMENT, "row_base needs offsets");
    if (num_tables < 1 || num_tables > 4096)
      return fail(CTR_ERR_UNSUPPORTED, "num_tables %d out of [1, 4096]", num_tables);
    if (batch < 0 || (int64_t)num_tables * batch > kMaxElems)
      return fail(CTR_ERR_INVALID_ARGUMENT, "bad batch %lld", (long long)batch);
    if (total_rows < 1) return fail(CTR_ERR_INVALID_ARGUMENT, "total_rows must be >= 1");
  }
  if (max_table_rows < 0) return fail(CTR_ERR_INVALID_ARGUMENT, "max_table_rows < 0");
  const size_t need = ctr::unique_workspace_bytes(n);
  if (!workspace) {
    *workspace_bytes = need;
    return CTR_OK;
  }
  if (*workspace_bytes < need)
    return fail(CTR_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", *workspace_bytes, need);
  if (!aligned16(workspace)) return fail(CTR_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
  if (!num_unique) return fail(CTR_ERR_INVALID_ARGUMENT, "num_unique is NULL");
  if (n > 0 && (!ids || !uniq))
    return fail(CTR_ERR_INVALID_ARGUMENT, "ids and uniq are required");
  if (sorted_src && (reinterpret_cast<uintptr_t>(sorted_src) & src_align(src_layout)))
    return fail(CTR_ERR_UNSUPPORTED, "sorted_src is not %d-byte aligned",
                (int)src_align(src_layout) + 1);
  int bits;
  bool is_signed = false;
  if (row_base) {
    bits = bitlen((uint64_t)(total_rows - 1));
  } else if (key_modulus > 0) {
    bits = bitlen((uint64_t)(key_modulus - 1));
  } else {
    bits = 64;
    is_signed = true;
  }
  if (bits < 1) bits = 1;
  // Tables as segments: sort the local row bits within each table when that takes fewer
  // passes of at most 8 bits than the global key, and (t << L) | local fits 32 bits.
  int seg_bits = 0;
  if (row_base && max_table_rows > 0 && num_tables >= 2 && num_tables <= 512 &&
      key_modulus == 0) {
    const int L = max_table_rows > 1 ? bitlen((uint64_t)(max_table_rows - 1)) : 1;
    if (L + bitlen((uint64_t)(num_tables - 1)) <= 32 && (L + 7) / 8 < (bits + 7) / 8)
      seg_bits = L;
  }
  return hip_status(ctr::launch_unique(ids, id_type == CTR_I64, n, offsets, batch, num_tables,
                                       row_base, key_modulus, bits, seg_bits, is_signed, uniq,
                                       inverse,
                                       num_unique, perm, seg_offsets, sorted_src,
                                       src_layout == CTR_SRC_ROWS, workspace,
                                       (hipStream_t)stream),
                    "ctr_unique_ids");
}

int32_t ctr_gather_rows(const void* table, int32_t dtype, int64_t total_rows, int32_t dim,
                        const int64_t* rows, const int32_t* num_rows, int64_t capacity,
                        float* out, void* stream) {
  g_msg[0] = 0;
  int32_t st = check_table(table, dtype, total_rows, dim);
  if (st) return st;
  if (capacity < 0 || capacity > kMaxElems) return fail(CTR_ERR_INVALID_ARGUMENT, "bad capacity");
  if (capacity > 0 && (!rows || !num_rows || !out))
    return fail(CTR_ERR_INVALID_ARGUMENT, "rows, num_rows and out are required");
  if (out && !aligned16(out)) return fail(CTR_ERR_UNSUPPORTED, "out is not 16-byte aligned");
  return hip_status(ctr::launch_gather_rows(table, dtype, total_rows, dim, rows,
                                            num_rows, capacity, out, (hipStream_t)stream),
                    "ctr_gather_rows");
}

int32_t ctr_embbag_fwd(const void* table, int32_t dtype, int64_t total_rows, int32_t dim,
                       const int64_t* row_base, int32_t num_tables, const void* indices,
                       int32_t index_type, int64_t nnz, const int64_t* offsets, int64_t batch,
                       void* out, int32_t out_dtype, int64_t out_stride_b, int64_t out_stride_t,
                       void* workspace, size_t* workspace_bytes, void* stream) {
  g_msg[0] = 0;
  if (!workspace_bytes) return fail(CTR_ERR_INVALID_ARGUMENT, "workspace_bytes is NULL");
  if (out_dtype != CTR_F32 && out_dtype != CTR_BF16)
    return fail(CTR_ERR_INVALID_ARGUMENT, "out_dtype %d is not CTR_F32 or CTR_BF16", out_dtype);
  if (nnz < 0 || nnz > kMaxElems) return fail(CTR_ERR_INVALID_ARGUMENT, "bad nnz");
  if (dim <= 0 || dim > 4096) return fail(CTR_ERR_INVALID_ARGUMENT, "bad dim %d", dim);
  const size_t need = ctr::embbag_fwd_workspace_bytes(nnz, dim);
  if (!workspace) {                       // the query needs only nnz and dim
    *workspace_bytes = need;
    return CTR_OK;
  }
  int32_t st = check_table(table, dtype, total_rows, dim);
  if (st) return st;
  if (*workspace_bytes < need)
    return fail(CTR_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", *workspace_bytes, need);
  if (!aligned16(workspace)) return fail(CTR_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
  if (index_type != CTR_I32 && index_type != CTR_I64)
    return fail(CTR_ERR_INVALID_ARGUMENT, "index_type %d is not CTR_I32 or CTR_I64", index_type);
  if (num_tables < 1) return fail(CTR_ERR_INVALID_ARGUMENT, "num_tables must be >= 1");
  if (batch < 0 || (int64_t)num_tables * batch > kMaxElems)
    return fail(CTR_ERR_INVALID_ARGUMENT, "bad batch %lld", (long long)batch);
  if (nnz < 0 || nnz > kMaxElems) return fail(CTR_ERR_INVALID_ARGUMENT, "bad nnz");
  if (!offsets || !out) return fail(CTR_ERR_INVALID_ARGUMENT, "offsets and out are required");
  if (nnz > 0 && !indices) return fail(CTR_ERR_INVALID_ARGUMENT, "indices is NULL");
  if (out_stride_b < 0 || out_stride_t < 0)
    return fail(CTR_ERR_INVALID_ARGUMENT, "negative output stride");
  if (num_tables > 1 && out_stride_t < dim && out_stride_b < dim)
    return fail(CTR_ERR_INVALID_ARGUMENT, "output strides smaller than dim");
  // fp32 vectors go out in 16-byte pieces of 4 values, bf16 ones in pieces of up to 8
  const int64_t sm = out_dtype == CTR_BF16 ? 8 : 4;
  if (!aligned16(out) || out_stride_b % sm || out_stride_t % sm)
    return fail(CTR_ERR_UNSUPPORTED, "out must be 16-byte aligned with strides multiple of %d",
                (int)sm);
  return hip_status(ctr::launch_embbag_fwd(table, dtype, total_rows, dim, row_base,
                                           num_tables, indices, index_type == CTR_I64, nnz,
                                           offsets, batch, out, out_dtype == CTR_BF16,
                                           out_stride_b, out_stride_t, workspace,
                                           (hipStream_t)stream),
                    "ctr_embbag_fwd");
}

int32_t ctr_embbag_bwd(const float* grad, int64_t grad_stride_b, int64_t grad_stride_t,
                       const int64_t* offsets, int64_t batch, int32_t num_tables, int32_t dim,
                       int64_t nnz, const int32_t* perm, const int32_t* inverse,
                       const int32_t* sorted_src, const int32_t* num_unique, float* row_grads,
                       void* workspace, size_t* workspace_bytes, void* stream) {
  g_msg[0] = 0;
  if (!workspace_bytes) return fail(CTR_ERR_INVALID_ARGUMENT, "workspace_bytes is NULL");
  if (dim <= 0) return fail(CTR_ERR_INVALID_ARGUMENT, "dim must be positive");
  if (dim % 4) return fail(CTR_ERR_UNSUPPORTED, "dim %d is not a multiple of 4", dim);
  if (dim > 1024) return fail(CTR_ERR_UNSUPPORTED, "dim %d above 1024", dim);
  if (nnz < 0 || nnz > kMaxElems) return fail(CTR_ERR_INVALID_ARGUMENT, "bad nnz");
  if (num_tables < 1) return fail(CTR_ERR_INVALID_ARGUMENT, "num_tables must be >= 1");
  if (batch < 0 || (int64_t)num_tables * batch > kMaxElems)
    return fail(CTR_ERR_INVALID_ARGUMENT, "bad batch");
  if (nnz > 0 && batch == 0)
    return fail(CTR_ERR_INVALID_ARGUMENT, "nnz > 0 needs at least one bag");
  const size_t need = ctr::embbag_bwd_workspace_bytes(nnz, dim);
  if (!workspace) {
    *workspace_bytes = need;
    return CTR_OK;
  }
  if (*workspace_bytes < need)
    return fail(CTR_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", *workspace_bytes, need);
  if (!offsets || !num_unique) return fail(CTR_ERR_INVALID_ARGUMENT, "offsets and num_unique are required");
  if (nnz > 0 && (!grad || !row_grads))
    return fail(CTR_ERR_INVALID_ARGUMENT, "grad and row_grads are required");
  if (nnz > 0 && !sorted_src && (!perm || !inverse))
    return fail(CTR_ERR_INVALID_ARGUMENT, "either sorted_src or perm and inverse are required");
  if (sorted_src && (reinterpret_cast<uintptr_t>(sorted_src) & 15u))
    return fail(CTR_ERR_UNSUPPORTED, "sorted_src is not 16-byte aligned");
  if (grad_stride_b < 0 || grad_stride_t < 0)
    return fail(CTR_ERR_INVALID_ARGUMENT, "negative gradient stride");
  if ((grad && !aligned16(grad)) || (row_grads && !aligned16(row_grads)) || grad_stride_b % 4 ||
      grad_stride_t % 4)
    return fail(CTR_ERR_UNSUPPORTED, "grad/row_grads must be 16-byte aligned, strides multiple of 4");
  if (!aligned16(workspace)) return fail(CTR_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
  return hip_status(ctr::launch_embbag_bwd(grad, false, grad_stride_b, grad_stride_t, offsets,
                                           batch, num_tables, dim, nnz, perm, inverse,
                                           sorted_src, false, num_unique, row_grads, nullptr, 0,
                                           0, nullptr, 0.f, 0, workspace, (hipStream_t)stream),
                    "ctr_embbag_bwd");
}

static int32_t embbag_bwd_sgd_common(const void* grad, bool grad_bf16, int64_t grad_stride_b,
                                     int64_t grad_stride_t, const int64_t* offsets,
                                     int64_t batch, int32_t num_tables, int64_t nnz,
                                     const int32_t* sorted_src, int32_t src_layout,
                                     const int32_t* num_unique,
                                     void* table, int32_t dtype, int64_t total_rows, int32_t dim,
                                     const int64_t* uniq, float lr, float* row_grads,
                                     void* workspace, size_t* workspace_bytes, bool stochastic,
                                     uint64_t seed, void* stream, const char* name,
                                     void* l0_begin = nullptr, void* l0_end = nullptr,
                                     bool noalloc = false) {
  g_msg[0] = 0;
  if (!noalloc && !workspace_bytes)
    return fail(CTR_ERR_INVALID_ARGUMENT, "workspace_bytes is NULL");
  if (table) {
    int32_t st = check_table(table, dtype, total_rows, dim);
    if (st) return st;
  } else {
    if (dim <= 0) return fail(CTR_ERR_INVALID_ARGUMENT, "dim must be positive");
    if (dim % 4) return fail(CTR_ERR_UNSUPPORTED, "dim %d is not a multiple of 4", dim);
    if (stochastic) return fail(CTR_ERR_INVALID_ARGUMENT, "stochastic rounding needs a table");
  }
  if (stochastic && dtype == CTR_F32)
    return fail(CTR_ERR_UNSUPPORTED, "stochastic rounding needs a CTR_BF16 or CTR_F16 table");
  if (dim > 1024) return fail(CTR_ERR_UNSUPPORTED, "dim %d above 1024", dim);
  if (nnz < 0 || nnz > kMaxElems) return fail(CTR_ERR_INVALID_ARGUMENT, "bad nnz");
  if (num_tables < 1) return fail(CTR_ERR_INVALID_ARGUMENT, "num_tables must be >= 1");
  if (batch < 0 || (int64_t)num_tables * batch > kMaxElems)
    return fail(CTR_ERR_INVALID_ARGUMENT, "bad batch");
  if (nnz > 0 && batch == 0)
    return fail(CTR_ERR_INVALID_ARGUMENT, "nnz > 0 needs at least one bag");
  if (noalloc) {
    const size_t need = ctr::embbag_bwd_noalloc_bytes(nnz, dim);
    if (need > ctr::kNoallocScratchBytes)
      return fail(CTR_ERR_UNSUPPORTED,
                  "nnz %lld, dim %d need %zu bytes of scratch, above the %zu of %s",
                  (long long)nnz, dim, need, ctr::kNoallocScratchBytes, name);
  } else {
    const size_t need = ctr::embbag_bwd_workspace_bytes(nnz, dim);
    if (!workspace) {
      *workspace_bytes = need;
      return CTR_OK;
    }
    if (*workspace_bytes < need)
      return fail(CTR_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", *workspace_bytes,
                  need);
  }
  if (!offsets || !num_unique) return fail(CTR_ERR_INVALID_ARGUMENT, "offsets and num_unique are required");
  const bool rows = src_layout == CTR_SRC_ROWS;
  if (rows && (!table || row_grads))
    return fail(CTR_ERR_INVALID_ARGUMENT,
                "CTR_SRC_ROWS entries need a table and no row_grads (they carry no u)");
  if (rows && total_rows > kMaxElems)
    return fail(CTR_ERR_UNSUPPORTED, "CTR_SRC_ROWS needs total_rows below 2^31");
  if (nnz > 0 && (!grad || !sorted_src || (table && !rows && !uniq)))
    return fail(CTR_ERR_INVALID_ARGUMENT, "grad, sorted_src and uniq are required");
  if (!table && !row_grads)
    return fail(CTR_ERR_INVALID_ARGUMENT, "without a table, row_grads is required");
  if (!std::isfinite(lr)) return fail(CTR_ERR_INVALID_ARGUMENT, "lr is not finite");
  if (grad_stride_b < 0 || grad_stride_t < 0)
    return fail(CTR_ERR_INVALID_ARGUMENT, "negative gradient stride");
  // bf16 rows are read 8 bytes per 4 columns, fp32 rows 16 bytes
  const uintptr_t galign = grad_bf16 ? 7u : 15u;
  if ((grad && (reinterpret_cast<uintptr_t>(grad) & galign)) ||
      (row_grads && !aligned16(row_grads)) || grad_stride_b % 4 || grad_stride_t % 4)
    return fail(CTR_ERR_UNSUPPORTED,
                "grad must be %d-byte aligned, row_grads 16-byte, strides multiple of 4",
                grad_bf16 ? 8 : 16);
  if (reinterpret_cast<uintptr_t>(sorted_src) & src_align(src_layout))
    return fail(CTR_ERR_UNSUPPORTED, "sorted_src is not %d-byte aligned",
                (int)src_align(src_layout) + 1);
  if (!noalloc && !aligned16(workspace))
    return fail(CTR_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
  const int mode = !table               ? 0
                   : dtype == CTR_BF16 ? (stochastic ? 3 : 2)
                   : dtype == CTR_F16  ? (stochastic ? 5 : 4)
                                       : 1;
  if (noalloc)
    return hip_status(ctr::launch_embbag_bwd_noalloc(
                          grad, grad_bf16, grad_stride_b, grad_stride_t, offsets, batch,
                          num_tables, dim, nnz, sorted_src, rows, row_grads, table, mode,
                          total_rows, uniq, lr, seed, (hipStream_t)stream),
                      name);
  return hip_status(ctr::launch_embbag_bwd(grad, grad_bf16, grad_stride_b, grad_stride_t,
                                           offsets, batch, num_tables, dim, nnz, nullptr,
                                           nullptr, sorted_src, rows,
                                           num_unique, row_grads, table, mode, total_rows, uniq,
                                           lr, seed, workspace, (hipStream_t)stream, l0_begin,
                                           l0_end),
                    name);
}

// The dtype and rounding codes of the public entry points, checked once for all of them.
static int32_t embbag_bwd_sgd_coded(const void* grad, int32_t grad_dtype, int64_t grad_stride_b,
                                    int64_t grad_stride_t, const int64_t* offsets, int64_t batch,
                                    int32_t num_tables, int64_t nnz, const int32_t* sorted_src,
                                    int32_t src_layout, const int32_t* num_unique, void* table,
                                    int32_t dtype, int64_t total_rows, int32_t dim,
                                    const int64_t* uniq, float lr, int32_t rounding,
                                    uint64_t seed, float* row_grads, void* workspace,
                                    size_t* workspace_bytes, void* stream, const char* name,
                                    void* l0_begin, void* l0_end, bool noalloc) {
  if (grad_dtype != CTR_F32 && grad_dtype != CTR_BF16) {
    g_msg[0] = 0;
    return fail(CTR_ERR_INVALID_ARGUMENT, "grad_dtype %d is not CTR_F32 or CTR_BF16", grad_dtype);
  }
  if (rounding != CTR_ROUND_NEAREST && rounding != CTR_ROUND_STOCHASTIC) {
    g_msg[0] = 0;
    return fail(CTR_ERR_INVALID_ARGUMENT, "unknown rounding %d", rounding);
  }
  if (src_layout != CTR_SRC_FULL && src_layout != CTR_SRC_ROWS) {
    g_msg[0] = 0;
    return fail(CTR_ERR_INVALID_ARGUMENT, "src_layout %d is not CTR_SRC_FULL or CTR_SRC_ROWS",
                src_layout);
  }
  return embbag_bwd_sgd_common(grad, grad_dtype == CTR_BF16, grad_stride_b, grad_stride_t,
                               offsets, batch, num_tables, nnz, sorted_src, src_layout,
                               num_unique, table,
                               dtype, total_rows, dim, uniq, lr, row_grads, workspace,
                               workspace_bytes, rounding == CTR_ROUND_STOCHASTIC, seed, stream,
                               name, l0_begin, l0_end, noalloc);
}

}  // extern "C"

namespace ctr {
// ctr_embbag_bwd_sgd with timing marks recorded right before and after the first
// reduce-by-key kernel (the native step runner's marks).
int32_t embbag_bwd_sgd_marked(const void* grad, int32_t grad_dtype, int64_t grad_stride_b,
                              int64_t grad_stride_t, const int64_t* offsets, int64_t batch,
                              int32_t num_tables, int64_t nnz, const int32_t* sorted_src,
                              int32_t src_layout, const int32_t* num_unique, void* table,
                              int32_t dtype, int64_t total_rows, int32_t dim,
                              const int64_t* uniq, float lr, int32_t rounding, uint64_t seed,
                              float* row_grads, void* workspace, size_t* workspace_bytes,
                              void* stream, void* l0_begin, void* l0_end) {
  return embbag_bwd_sgd_coded(grad, grad_dtype, grad_stride_b, grad_stride_t, offsets, batch,
                              num_tables, nnz, sorted_src, src_layout, num_unique, table, dtype,
                              total_rows,
                              dim, uniq, lr, rounding, seed, row_grads, workspace,
                              workspace_bytes, stream, "ctr_step_run (backward)", l0_begin,
                              l0_end, false);
}
}  // namespace ctr

extern "C" {

int32_t ctr_embbag_bwd_sgd(const void* grad, int32_t grad_dtype, int64_t grad_stride_b,
                           int64_t grad_stride_t, const int64_t* offsets, int64_t batch,
                           int32_t num_tables, int64_t nnz, const int32_t* sorted_src,
                           int32_t src_layout, const int32_t* num_unique, void* table,
                           int32_t dtype, int64_t total_rows, int32_t dim, const int64_t* uniq,
                           float lr, int32_t rounding, uint64_t seed, float* row_grads,
                           void* workspace, size_t* workspace_bytes, void* stream) {
  return embbag_bwd_sgd_coded(grad, grad_dtype, grad_stride_b, grad_stride_t, offsets, batch,
                              num_tables, nnz, sorted_src, src_layout, num_unique, table, dtype,
                              total_rows,
                              dim, uniq, lr, rounding, seed, row_grads, workspace,
                              workspace_bytes, stream, "ctr_embbag_bwd_sgd", nullptr, nullptr,
                              false);
}

int32_t ctr_embbag_bwd_sgd_noalloc(const void* grad, int32_t grad_dtype, int64_t grad_stride_b,
                                   int64_t grad_stride_t, const int64_t* offsets, int64_t batch,
                                   int32_t num_tables, int64_t nnz, const int32_t* sorted_src,
                                   int32_t src_layout, const int32_t* num_unique, void* table,
                                   int32_t dtype, int64_t total_rows, int32_t dim,
                                   const int64_t* uniq, float lr, int32_t rounding,
                                   uint64_t seed, float* row_grads, void* stream) {
  return embbag_bwd_sgd_coded(grad, grad_dtype, grad_stride_b, grad_stride_t, offsets, batch,
                              num_tables, nnz, sorted_src, src_layout, num_unique, table, dtype,
                              total_rows,
                              dim, uniq, lr, rounding, seed, row_grads, nullptr, nullptr, stream,
                              "ctr_embbag_bwd_sgd_noalloc", nullptr, nullptr, true);
}

size_t ctr_embbag_bwd_noalloc_scratch_bytes(int64_t nnz, int32_t dim) {
  if (nnz < 0 || dim <= 0 || dim % 4) return (size_t)-1;
  return ctr::embbag_bwd_noalloc_bytes(nnz, dim);
}

size_t ctr_noalloc_scratch_capacity(void) { return ctr::kNoallocScratchBytes; }

static int32_t sparse_sgd_common(void* table, int32_t dtype, int64_t total_rows, int32_t dim,
                                 const int64_t* uniq, const int32_t* num_unique,
                                 int64_t capacity, const float* row_grads, float lr,
                                 bool stochastic, uint64_t seed, void* stream, const char* name) {
  g_msg[0] = 0;
  int32_t st = check_table(table, dtype, total_rows, dim);
  if (st) return st;
  if (stochastic && dtype == CTR_F32)
    return fail(CTR_ERR_UNSUPPORTED, "stochastic rounding needs a CTR_BF16 or CTR_F16 table");
  if (capacity < 0 || capacity > kMaxElems) return fail(CTR_ERR_INVALID_ARGUMENT, "bad capacity");
  if (capacity > 0 && (!uniq || !num_unique || !row_grads))
    return fail(CTR_ERR_INVALID_ARGUMENT, "uniq, num_unique and row_grads are required");
  if (!std::isfinite(lr)) return fail(CTR_ERR_INVALID_ARGUMENT, "lr is not finite");
  if (row_grads && !aligned16(row_grads))
    return fail(CTR_ERR_UNSUPPORTED, "row_grads is not 16-byte aligned");
  return hip_status(ctr::launch_sparse_sgd(table, dtype, total_rows, dim, uniq,
                                           num_unique, capacity, row_grads, lr, stochastic, seed,
                                           (hipStream_t)stream),
                    name);
}

int32_t ctr_sparse_sgd(void* table, int32_t dtype, int64_t total_rows, int32_t dim,
                       const int64_t* uniq, const int32_t* num_unique, int64_t capacity,
                       const float* row_grads, float lr, int32_t rounding, uint64_t seed,
                       void* stream) {
  if (rounding != CTR_ROUND_NEAREST && rounding != CTR_ROUND_STOCHASTIC) {
    g_msg[0] = 0;
    return fail(CTR_ERR_INVALID_ARGUMENT, "unknown rounding %d", rounding);
  }
  return sparse_sgd_common(table, dtype, total_rows, dim, uniq, num_unique, capacity, row_grads,
                           lr, rounding == CTR_ROUND_STOCHASTIC, seed, stream, "ctr_sparse_sgd");
}

uint64_t ctr_sr_step_seed(uint64_t base, int64_t k) {
  uint64_t z = base + (uint64_t)(k + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// pairs: ctr::kPairStrict, kPairSelf or kPairGram (the interaction's pair set).
static int32_t check_interaction(const float* Z, int64_t batch, int32_t F, int32_t dim,
                                 int32_t compute, int pairs, const float* out, int64_t stride) {
  if (batch < 0 || batch > kMaxElems) return fail(CTR_ERR_INVALID_ARGUMENT, "bad batch");
  const int fmin = pairs == ctr::kPairStrict ? 2 : 1;
  if (F < fmin)
    return fail(CTR_ERR_INVALID_ARGUMENT, "num_vectors must be >= %d (got %d)", fmin, F);
  if (F > 4096) return fail(CTR_ERR_UNSUPPORTED, "num_vectors %d above 4096", F);
  if (dim <= 0) return fail(CTR_ERR_INVALID_ARGUMENT, "dim must be positive");
  if (compute != CTR_F32 && compute != CTR_BF16)
    return fail(CTR_ERR_INVALID_ARGUMENT, "compute %d is not CTR_F32 or CTR_BF16", compute);
  if (batch > 0 && (!Z || !out)) return fail(CTR_ERR_INVALID_ARGUMENT, "Z and output are required");
  const int64_t P = pairs == ctr::kPairGram   ? (int64_t)F * F
                    : pairs == ctr::kPairSelf ? (int64_t)F * (F + 1) / 2
                                              : (int64_t)F * (F - 1) / 2;
  if (stride < dim + P) return fail(CTR_ERR_INVALID_ARGUMENT, "stride %lld < dim + P", (long long)stride);
  if (compute == CTR_BF16) {
    if (!ctr::interaction_bf16_supported(F, dim, pairs))
      return fail(CTR_ERR_UNSUPPORTED, "bf16 path needs dim in {16,32,64,128}, F <= 128");
    if (Z && !aligned16(Z)) return fail(CTR_ERR_UNSUPPORTED, "Z is not 16-byte aligned");
  } else if (!ctr::interaction_f32_supported(F, dim, pairs)) {
    return fail(CTR_ERR_UNSUPPORTED, "fp32 path: one sample of F=%d, dim=%d exceeds 64 KiB of LDS", F, dim);
  }
  return CTR_OK;
}

// A bf16 Z (z_dtype CTR_BF16): the matrix-core interaction of the strict pairs only.
static int32_t check_z_dtype(int32_t z_dtype, int32_t compute, int pairs) {
  if (z_dtype != CTR_F32 && z_dtype != CTR_BF16)
    return fail(CTR_ERR_INVALID_ARGUMENT, "z_dtype %d is not CTR_F32 or CTR_BF16", z_dtype);
  if (z_dtype == CTR_BF16 && (compute != CTR_BF16 || pairs != ctr::kPairStrict))
    return fail(CTR_ERR_UNSUPPORTED,
                "a bf16 Z needs compute = CTR_BF16 (the dot interaction on matrix cores)");
  return CTR_OK;
}

static int32_t interaction_fwd_common(const void* Z, int32_t z_dtype, int64_t batch, int32_t F,
                                      int32_t dim, int32_t compute, int pairs, float* R,
                                      int64_t r_stride, void* stream, const char* name) {
  g_msg[0] = 0;
  int32_t st = check_z_dtype(z_dtype, compute, pairs);
  if (st) return st;
  st = check_interaction(static_cast<const float*>(Z), batch, F, dim, compute, pairs, R,
                         r_stride);
  if (st) return st;
  return hip_status(ctr::launch_interaction_fwd(Z, z_dtype == CTR_BF16, batch, F, dim,
                                                compute == CTR_BF16, pairs, R, r_stride,
                                                (hipStream_t)stream),
                    name);
}

static int32_t interaction_bwd_common(const void* Z, int32_t z_dtype, const float* dR,
                                      int64_t dr_stride, int64_t batch, int32_t F, int32_t dim,
                                      int32_t compute, int pairs, int32_t dz_dtype, void* dZ,
                                      void* stream, const char* name) {
  g_msg[0] = 0;
  if (dz_dtype != CTR_F32 && dz_dtype != CTR_BF16)
    return fail(CTR_ERR_INVALID_ARGUMENT, "dz_dtype %d is not CTR_F32 or CTR_BF16", dz_dtype);
  const bool dz_bf16 = dz_dtype == CTR_BF16;
  int32_t st = check_z_dtype(z_dtype, compute, pairs);
  if (st) return st;
  if (z_dtype == CTR_BF16 && !dz_bf16)
    return fail(CTR_ERR_UNSUPPORTED, "a bf16 Z takes a bf16 dZ");
  st = check_interaction(static_cast<const float*>(Z), batch, F, dim, compute, pairs,
                         static_cast<const float*>(dZ), dr_stride);
  if (st) return st;
  if (batch > 0 && !dR) return fail(CTR_ERR_INVALID_ARGUMENT, "dR is NULL");
  if (dz_bf16 && compute != CTR_BF16)
    return fail(CTR_ERR_UNSUPPORTED, "a bf16 dZ needs compute = CTR_BF16");
  if (compute == CTR_BF16 && dZ && !aligned16(dZ))
    return fail(CTR_ERR_UNSUPPORTED, "dZ is not 16-byte aligned");
  return hip_status(ctr::launch_interaction_bwd(Z, z_dtype == CTR_BF16, dR, dr_stride, batch, F,
                                                dim, compute == CTR_BF16, pairs, dz_bf16, dZ,
                                                (hipStream_t)stream),
                    name);
}

int32_t ctr_dot_interaction_fwd(const void* Z, int32_t z_dtype, int64_t batch,
                                int32_t num_vectors, int32_t dim, int32_t compute, float* R,
                                int64_t r_stride, void* stream) {
  return interaction_fwd_common(Z, z_dtype, batch, num_vectors, dim, compute, ctr::kPairStrict,
                                R, r_stride, stream, "ctr_dot_interaction_fwd");
}

int32_t ctr_embbag_interaction_fwd(const void* table, int32_t dtype, int64_t total_rows,
                                   int32_t dim, const int64_t* row_base, int32_t num_tables,
                                   const void* indices, int32_t index_type, int64_t nnz,
                                   const int64_t* offsets, int64_t batch, float* Z,
                                   int32_t compute, float* R, int64_t r_stride, void* stream) {
  g_msg[0] = 0;
  int32_t st = check_table(table, dtype, total_rows, dim);
  if (st) return st;
  if (dtype == CTR_F16)
    return fail(CTR_ERR_UNSUPPORTED,
                "CTR_F16 tables: ctr_embbag_fwd then ctr_dot_interaction_fwd");
  if (index_type != CTR_I32 && index_type != CTR_I64)
    return fail(CTR_ERR_INVALID_ARGUMENT, "index_type %d is not CTR_I32 or CTR_I64", index_type);
  if (num_tables < 1) return fail(CTR_ERR_INVALID_ARGUMENT, "num_tables must be >= 1");
  if (batch < 0 || (int64_t)num_tables * batch > kMaxElems ||
      batch * (num_tables + 1) * (int64_t)dim > ((int64_t)1 << 40))
    return fail(CTR_ERR_INVALID_ARGUMENT, "bad batch %lld", (long long)batch);
  if (nnz < 0 || nnz > kMaxElems) return fail(CTR_ERR_INVALID_ARGUMENT, "bad nnz");
  if (compute != CTR_F32 && compute != CTR_BF16)
    return fail(CTR_ERR_INVALID_ARGUMENT, "compute %d is not CTR_F32 or CTR_BF16", compute);
  if (batch > 0 && (!offsets || !Z || !R))
    return fail(CTR_ERR_INVALID_ARGUMENT, "offsets, Z and R are required");
  if (nnz > 0 && !indices) return fail(CTR_ERR_INVALID_ARGUMENT, "indices is NULL");
  const int64_t F = (int64_t)num_tables + 1;
  if (r_stride < dim + F * (F - 1) / 2)
    return fail(CTR_ERR_INVALID_ARGUMENT, "r_stride %lld < dim + P", (long long)r_stride);
  if (Z && !aligned16(Z)) return fail(CTR_ERR_UNSUPPORTED, "Z is not 16-byte aligned");
  if (!ctr::embbag_interaction_supported(num_tables, dim, dtype == CTR_BF16, compute == CTR_BF16))
    return fail(CTR_ERR_UNSUPPORTED,
                "fused shape: dim/(values per 16 bytes) a power of two <= 32, num_tables <= 256, "
                "one sample's pooled copy <= 46 KiB; bf16 compute: dim in {16,32,64,128}, F <= 128");
  return hip_status(ctr::launch_embbag_interaction_fwd(table, dtype == CTR_BF16, total_rows, dim,
                                                       row_base, num_tables, indices,
                                                       index_type == CTR_I64, nnz, offsets, batch,
                                                       Z, compute == CTR_BF16, R, r_stride,
                                                       (hipStream_t)stream),
                    "ctr_embbag_interaction_fwd");
}

int32_t ctr_dot_interaction_bwd(const void* Z, int32_t z_dtype, const float* dR,
                                int64_t dr_stride, int64_t batch, int32_t num_vectors,
                                int32_t dim, int32_t compute, int32_t dz_dtype, void* dZ,
                                void* stream) {
  return interaction_bwd_common(Z, z_dtype, dR, dr_stride, batch, num_vectors, dim, compute,
                                ctr::kPairStrict, dz_dtype, dZ, stream, "ctr_dot_interaction_bwd");
}

int32_t ctr_dot_interaction_self_fwd(const float* Z, int64_t batch, int32_t num_vectors,
                                     int32_t dim, int32_t compute, float* R, int64_t r_stride,
                                     void* stream) {
  return interaction_fwd_common(Z, CTR_F32, batch, num_vectors, dim, compute, ctr::kPairSelf, R,
                                r_stride, stream, "ctr_dot_interaction_self_fwd");
}

int32_t ctr_dot_interaction_self_bwd(const float* Z, const float* dR, int64_t dr_stride,
                                     int64_t batch, int32_t num_vectors, int32_t dim,
                                     int32_t compute, int32_t dz_dtype, void* dZ, void* stream) {
  return interaction_bwd_common(Z, CTR_F32, dR, dr_stride, batch, num_vectors, dim, compute,
                                ctr::kPairSelf, dz_dtype, dZ, stream,
                                "ctr_dot_interaction_self_bwd");
}

int32_t ctr_dot_interaction_gram_fwd(const float* Z, int64_t batch, int32_t num_vectors,
                                     int32_t dim, int32_t compute, float* R, int64_t r_stride,
                                     void* stream) {
  return interaction_fwd_common(Z, CTR_F32, batch, num_vectors, dim, compute, ctr::kPairGram, R,
                                r_stride, stream, "ctr_dot_interaction_gram_fwd");
}

int32_t ctr_dot_interaction_gram_bwd(const float* Z, const float* dR, int64_t dr_stride,
                                     int64_t batch, int32_t num_vectors, int32_t dim,
                                     int32_t compute, int32_t dz_dtype, void* dZ, void* stream) {
  return interaction_bwd_common(Z, CTR_F32, dR, dr_stride, batch, num_vectors, dim, compute,
                                ctr::kPairGram, dz_dtype, dZ, stream,
                                "ctr_dot_interaction_gram_bwd");
}

static int32_t check_fm(const float* Z, int64_t batch, int32_t F, int32_t dim, const float* a,
                        const float* b) {
  if (batch < 0 || batch > kMaxElems) return fail(CTR_ERR_INVALID_ARGUMENT, "bad batch");
  if (F < 1) return fail(CTR_ERR_INVALID_ARGUMENT, "num_vectors must be >= 1 (got %d)", F);
  if (dim <= 0) return fail(CTR_ERR_INVALID_ARGUMENT, "dim must be positive");
  if ((int64_t)F * dim > kMaxElems) return fail(CTR_ERR_INVALID_ARGUMENT, "F * dim too large");
  if (batch > 0 && (!Z || !a || !b))
    return fail(CTR_ERR_INVALID_ARGUMENT, "Z and the other arrays are required");
  return CTR_OK;
}

int32_t ctr_fm_interaction_fwd(const float* Z, int64_t batch, int32_t num_vectors, int32_t dim,
                               float* out, void* stream) {
  g_msg[0] = 0;
  int32_t st = check_fm(Z, batch, num_vectors, dim, out, out);
  if (st) return st;
  return hip_status(ctr::launch_fm_fwd(Z, batch, num_vectors, dim, out, (hipStream_t)stream),
                    "ctr_fm_interaction_fwd");
}

int32_t ctr_fm_interaction_bwd(const float* Z, const float* dout, int64_t batch,
                               int32_t num_vectors, int32_t dim, float* dZ, void* stream) {
  g_msg[0] = 0;
  int32_t st = check_fm(Z, batch, num_vectors, dim, dout, dZ);
  if (st) return st;
  return hip_status(ctr::launch_fm_bwd(Z, dout, batch, num_vectors, dim, dZ, (hipStream_t)stream),
                    "ctr_fm_interaction_bwd");
}

static bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int32_t ctr_dict_build(const int64_t* keys, const int32_t* rows, const int32_t* hot_slots,
                       int64_t n, void* slots, int64_t capacity, int32_t* status,
                       void* stream) {
  g_msg[0] = 0;
  if (n < 0 || n > kMaxElems) return fail(CTR_ERR_INVALID_ARGUMENT, "bad n");
  if (!pow2(capacity) || capacity < 2)
    return fail(CTR_ERR_INVALID_ARGUMENT, "capacity %lld is not a power of two >= 2",
                (long long)capacity);
  if (n >= capacity)
    return fail(CTR_ERR_INVALID_ARGUMENT, "n = %lld keys need capacity > n (got %lld)",
                (long long)n, (long long)capacity);
  if (!slots || !status) return fail(CTR_ERR_INVALID_ARGUMENT, "slots and status are required");
  if (n > 0 && (!keys || !rows)) return fail(CTR_ERR_INVALID_ARGUMENT, "keys and rows are required");
  if (!aligned16(slots)) return fail(CTR_ERR_UNSUPPORTED, "slots is not 16-byte aligned");
  return hip_status(ctr::launch_dict_build(keys, rows, hot_slots, n, slots, capacity, status,
                                           (hipStream_t)stream),
                    "ctr_dict_build");
}

int32_t ctr_dict_lookup(const int64_t* ids, int64_t n, const void* slots, int64_t capacity,
                        int64_t* values, void* stream) {
  g_msg[0] = 0;
  if (n < 0 || n > kMaxElems) return fail(CTR_ERR_INVALID_ARGUMENT, "bad n");
  if (!pow2(capacity) || capacity < 2)
    return fail(CTR_ERR_INVALID_ARGUMENT, "capacity %lld is not a power of two >= 2",
                (long long)capacity);
  if (n > 0 && (!ids || !slots || !values))
    return fail(CTR_ERR_INVALID_ARGUMENT, "ids, slots and values are required");
  if (slots && !aligned16(slots)) return fail(CTR_ERR_UNSUPPORTED, "slots is not 16-byte aligned");
  return hip_status(ctr::launch_dict_lookup(ids, n, slots, capacity, values, (hipStream_t)stream),
                    "ctr_dict_lookup");
}

int32_t ctr_dict_embbag_fwd(const int64_t* values, int64_t nnz, const int64_t* offsets,
                            int64_t batch, int32_t num_tables, const void* hot_rows,
                            int64_t num_hot, const void* table, int64_t num_rows, int32_t dtype,
                            int32_t dim, float* out, int64_t out_stride_b,
                            int64_t out_stride_t, void* stream) {
  g_msg[0] = 0;
  int32_t st = check_table(table, dtype, num_rows, dim);
  if (st) return st;
  if (num_rows < 1) return fail(CTR_ERR_INVALID_ARGUMENT, "the dictionary table needs >= 1 row");
  if (num_hot < 0) return fail(CTR_ERR_INVALID_ARGUMENT, "num_hot < 0");
  if (num_hot > 0 && !hot_rows) return fail(CTR_ERR_INVALID_ARGUMENT, "hot_rows is NULL");
  if (hot_rows && !aligned16(hot_rows))
    return fail(CTR_ERR_UNSUPPORTED, "hot_rows is not 16-byte aligned");
  if (nnz < 0 || nnz > kMaxElems) return fail(CTR_ERR_INVALID_ARGUMENT, "bad nnz");
  if (num_tables < 1) return fail(CTR_ERR_INVALID_ARGUMENT, "num_tables must be >= 1");
  if (batch < 0 || (int64_t)num_tables * batch > kMaxElems)
    return fail(CTR_ERR_INVALID_ARGUMENT, "bad batch");
  if (batch > 0 && (!offsets || !out)) return fail(CTR_ERR_INVALID_ARGUMENT, "offsets and out are required");
  if (nnz > 0 && !values) return fail(CTR_ERR_INVALID_ARGUMENT, "values is NULL");
  if (out && (!aligned16(out) || out_stride_b % 4 || out_stride_t % 4 || out_stride_b < 0 ||
              out_stride_t < 0))
    return fail(CTR_ERR_UNSUPPORTED, "out must be 16-byte aligned with strides multiple of 4");
  return hip_status(ctr::launch_dict_pool(values, nnz, offsets, batch, num_tables, hot_rows,
                                          num_hot, table, num_rows, dtype, dim, out,
                                          out_stride_b, out_stride_t, (hipStream_t)stream),
                    "ctr_dict_embbag_fwd");
}

int32_t ctr_init_tables_hash(void* table, int32_t dtype, int32_t dim, const int64_t* row_base_host,
                            int32_t num_tables, uint64_t seed, void* stream) {
  g_msg[0] = 0;
  if (!row_base_host || num_tables < 1)
    return fail(CTR_ERR_INVALID_ARGUMENT, "row_base_host and num_tables >= 1 are required");
  for (int32_t t = 0; t < num_tables; ++t)
    if (row_base_host[t + 1] < row_base_host[t] || row_base_host[0] != 0)
      return fail(CTR_ERR_INVALID_ARGUMENT, "row_base_host must start at 0 and not decrease");
  int32_t st = check_table(table, dtype, row_base_host[num_tables], dim);
  if (st) return st;
  for (int32_t t = 0; t < num_tables; ++t) {
    const int64_t rows = row_base_host[t + 1] - row_base_host[t];
    if (rows == 0) continue;
    const float scale = (float)(1.0 / std::sqrt((double)rows));
    hipError_t e = ctr::launch_init_table(table, dtype, dim, row_base_host[t], rows,
                                          scale, seed, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "ctr_init_tables_hash");
  }
  return CTR_OK;
}

// ---------------------------------------------------------------- dense layers and head
constexpr int32_t kMaxWidth = 65536;       // layer widths (inputs K, outputs N)

static int32_t check_dense(int64_t M, int32_t K, int32_t N, int32_t compute, int64_t x_stride,
                           int64_t y_stride) {
  if (M < 0 || M > kMaxElems) return fail(CTR_ERR_INVALID_ARGUMENT, "bad batch rows M");
  if (K < 1 || K > kMaxWidth || N < 1 || N > kMaxWidth)
    return fail(CTR_ERR_INVALID_ARGUMENT, "layer widths must be in [1, %d] (got K=%d, N=%d)",
                kMaxWidth, K, N);
  if (compute != CTR_F32 && compute != CTR_BF16)
    return fail(CTR_ERR_INVALID_ARGUMENT, "compute %d is not CTR_F32 or CTR_BF16", compute);
  if (x_stride < K) return fail(CTR_ERR_INVALID_ARGUMENT, "x_stride < K");
  if (y_stride < N) return fail(CTR_ERR_INVALID_ARGUMENT, "y_stride < N");
  // one work-item per element in the elementwise passes: keep every product below 2^31
  if (M * (int64_t)N > kMaxElems || M * (int64_t)K > kMaxElems ||
      (int64_t)N * (K + 1) > kMaxElems)
    return fail(CTR_ERR_INVALID_ARGUMENT, "M * N, M * K and N * (K + 1) must be below 2^31");
  return CTR_OK;
}

int32_t ctr_dense_fwd(const float* X, int64_t x_stride, int64_t M, int32_t K, const float* W,
                      const float* b, int32_t N, int32_t relu, int32_t compute, float* Y,
                      int64_t y_stride, void* stream) {
  g_msg[0] = 0;
  int32_t st = check_dense(M, K, N, compute, x_stride, y_stride);
  if (st) return st;
  if (M > 0 && (!X || !W || !Y)) return fail(CTR_ERR_INVALID_ARGUMENT, "X, W and Y are required");
  return hip_status(ctr::launch_dense_fwd(X, x_stride, M, K, W, b, N, relu != 0,
                                          compute == CTR_BF16, Y, y_stride,
                                          (hipStream_t)stream),
                    "ctr_dense_fwd");
}

int32_t ctr_dense_bwd_sgd(const float* X, int64_t x_stride, int64_t M, int32_t K, float* W,
                          float* b, int32_t N, int32_t relu, const float* Y, int64_t y_stride,
                          const void* dY, int32_t dy_dtype, int64_t dy_stride, int32_t compute,
                          float lr, float* dX, int64_t dx_stride, void* workspace,
                          size_t* workspace_bytes, void* stream) {
  g_msg[0] = 0;
  int32_t st = check_dense(M, K, N, compute, x_stride, y_stride);
  if (st) return st;
  if (dy_dtype != CTR_F32 && dy_dtype != CTR_BF16)
    return fail(CTR_ERR_INVALID_ARGUMENT, "dy_dtype %d is not CTR_F32 or CTR_BF16", dy_dtype);
  if (dy_stride < N) return fail(CTR_ERR_INVALID_ARGUMENT, "dy_stride < N");
  if (dX && dx_stride < K) return fail(CTR_ERR_INVALID_ARGUMENT, "dx_stride < K");
  if (!workspace_bytes) return fail(CTR_ERR_INVALID_ARGUMENT, "workspace_bytes is required");
  const size_t need = ctr::dense_bwd_workspace_bytes(M, N, K, b != nullptr, relu != 0,
                                                     compute == CTR_BF16);
  if (!workspace) {
    *workspace_bytes = need;
    return CTR_OK;
  }
  if (*workspace_bytes < need)
    return fail(CTR_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", need,
                *workspace_bytes);
  if (!aligned16(workspace)) return fail(CTR_ERR_UNSUPPORTED, "workspace is not 16-byte aligned");
  if (M > 0 && (!X || !W || !dY || (relu && !Y)))
    return fail(CTR_ERR_INVALID_ARGUMENT, "X, W, dY (and Y with relu) are required");
  return hip_status(ctr::launch_dense_bwd_sgd(X, x_stride, M, K, W, b, N, relu != 0, Y, y_stride,
                                              dY, dy_dtype == CTR_BF16, dy_stride,
                                              compute == CTR_BF16, lr, dX, dx_stride, workspace,
                                              (hipStream_t)stream),
                    "ctr_dense_bwd_sgd");
}

int32_t ctr_logistic_ne(const float* logits, int64_t logit_stride, const float* labels,
                        int64_t M, float* prob, float* dlogits, int64_t dl_stride, float* stats,
                        void* stream) {
  g_msg[0] = 0;
  if (M < 1 || M > kMaxElems) return fail(CTR_ERR_INVALID_ARGUMENT, "bad M (need >= 1)");
  if (logit_stride < 1 || (dlogits && dl_stride < 1))
    return fail(CTR_ERR_INVALID_ARGUMENT, "strides must be >= 1");
  if (!logits || !labels || !stats)
    return fail(CTR_ERR_INVALID_ARGUMENT, "logits, labels and stats are required");
  return hip_status(ctr::launch_logistic_ne(logits, logit_stride, labels, M, prob, dlogits,
                                            dl_stride, stats, (hipStream_t)stream),
                    "ctr_logistic_ne");
}

int32_t ctr_validate_csr(const void* indices, int32_t index_type, int64_t nnz,
                         const int64_t* offsets, int64_t batch, int32_t num_tables,
                         const int64_t* row_base, int64_t total_rows, int32_t* bad_count,
                         void* stream) {
  g_msg[0] = 0;
  if (index_type != CTR_I32 && index_type != CTR_I64)
    return fail(CTR_ERR_INVALID_ARGUMENT, "index_type %d is not CTR_I32 or CTR_I64", index_type);
  if (nnz < 0 || nnz > kMaxElems || batch < 0 || num_tables < 1 ||
      (int64_t)num_tables * batch > kMaxElems)
    return fail(CTR_ERR_INVALID_ARGUMENT, "bad sizes");
  if (!offsets || !bad_count || (nnz > 0 && !indices))
    return fail(CTR_ERR_INVALID_ARGUMENT, "offsets, bad_count and indices are required");
  return hip_status(ctr::launch_validate_csr(indices, index_type == CTR_I64, nnz, offsets, batch,
                                             num_tables, row_base, total_rows, bad_count,
                                             (hipStream_t)stream),
                    "ctr_validate_csr");
}

}  // extern "C"
