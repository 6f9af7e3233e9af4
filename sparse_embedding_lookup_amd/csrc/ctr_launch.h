// ctr_launch.h -- host declarations of the kernel launchers shared by the libctr sources
// (the device helpers are in ctr_internal.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ctr {

// ----------------------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Shapes are validated by the caller.

// unique.hip
size_t unique_workspace_bytes(int64_t n);
// seg_bits > 0: the table-segmented sort over seg_bits local row bits (row_base and offsets
// given, (num_tables - 1) << seg_bits below 2^32, at most 512 tables).  sorted_src: int4
// (u, bag, key words) per sorted position, or with src_rows int2 (key, bag) (keys below 2^31).
hipError_t launch_unique(const void* ids, bool ids64, int64_t n, const int64_t* offsets,
                         int64_t batch, int32_t num_tables, const int64_t* row_base,
                         int64_t modulus, int key_bits, int seg_bits, bool key_signed,
                         int64_t* uniq, int32_t* inverse, int32_t* num_unique, int32_t* perm,
                         int32_t* seg_offsets, void* sorted_src, bool src_rows,
                         void* workspace, hipStream_t s);

// embbag.hip (elt: the table's kElt code, ctr_internal.h)
// The pooling; workspace (embbag_fwd_workspace_bytes) holds the long bags' chunk partials.
size_t embbag_fwd_workspace_bytes(int64_t nnz, int dim);
hipError_t launch_embbag_fwd(const void* table, int elt, int64_t total_rows, int dim,
                             const int64_t* row_base, int32_t num_tables, const void* idx,
                             bool idx64, int64_t nnz, const int64_t* offsets, int64_t batch,
                             void* out, bool out_bf16, int64_t sb, int64_t st, void* workspace,
                             hipStream_t s);
hipError_t launch_gather_rows(const void* table, int elt, int64_t total_rows, int dim,
                              const int64_t* rows, const int32_t* num_rows, int64_t capacity,
                              float* out, hipStream_t s);
hipError_t launch_sparse_sgd(void* table, int elt, int64_t total_rows, int dim,
                             const int64_t* uniq, const int32_t* num_unique, int64_t capacity,
                             const float* g, float lr, bool stochastic, uint64_t seed,
                             hipStream_t s);
hipError_t launch_init_table(void* table, int elt, int dim, int64_t row_begin,
                             int64_t rows, float scale, uint64_t seed, hipStream_t s);
hipError_t launch_validate_csr(const void* idx, bool idx64, int64_t nnz, const int64_t* offsets,
                               int64_t batch, int32_t num_tables, const int64_t* row_base,
                               int64_t total_rows, int32_t* bad, hipStream_t s);

// segreduce.hip
size_t embbag_bwd_workspace_bytes(int64_t nnz, int dim);
// sorted_src: int4 (u, bag, row words), or with src_rows int2 (row, bag): then a table and
// no row_grads.
hipError_t launch_embbag_bwd(const void* grad, bool grad_bf16, int64_t sb, int64_t st,
                             const int64_t* offsets,
                             int64_t batch, int32_t num_tables, int dim, int64_t nnz,
                             const int32_t* perm, const int32_t* inverse, const void* sorted_src,
                             bool src_rows, const int32_t* num_unique, float* row_grads,
                             void* table,
                             int sgd_mode, int64_t total_rows, const int64_t* uniq, float lr,
                             uint64_t seed, void* workspace, hipStream_t s,
                             void* l0_begin = nullptr, void* l0_end = nullptr);
// The backward that allocates nothing: its carries and ticket live in a device array of
// kNoallocScratchBytes per GPU (segreduce.hip); sorted_src is required, and the caller checks
// embbag_bwd_noalloc_bytes(nnz, dim) <= kNoallocScratchBytes first.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
size_t embbag_bwd_noalloc_bytes(int64_t nnz, int dim);
hipError_t launch_embbag_bwd_noalloc(const void* grad, bool grad_bf16, int64_t sb, int64_t st,
                                     const int64_t* offsets, int64_t batch, int32_t num_tables,
                                     int dim, int64_t nnz, const void* sorted_src,
                                     bool src_rows, float* row_grads, void* table, int sgd_mode,
                                     int64_t total_rows, const int64_t* uniq, float lr,
                                     uint64_t seed, hipStream_t s);
// The fused backward + SGD entry (ctr_embbag_bwd_sgd) with timing marks around its first
// reduce-by-key kernel (capi.cpp).
int32_t embbag_bwd_sgd_marked(const void* grad, int32_t grad_dtype, int64_t grad_stride_b,
                              int64_t grad_stride_t, const int64_t* offsets, int64_t batch,
                              int32_t num_tables, int64_t nnz, const int32_t* sorted_src,
                              int32_t src_layout, const int32_t* num_unique, void* table,
                              int32_t dtype, int64_t total_rows, int32_t dim,
                              const int64_t* uniq, float lr, int32_t rounding, uint64_t seed,
                              float* row_grads, void* workspace, size_t* workspace_bytes,
                              void* stream, void* l0_begin, void* l0_end);

// dict.hip
hipError_t launch_dict_build(const int64_t* keys, const int32_t* rows, const int32_t* hot_slots,
                             int64_t n, void* slots, int64_t capacity, int32_t* status,
                             hipStream_t s);
hipError_t launch_dict_lookup(const int64_t* ids, int64_t n, const void* slots,
                              int64_t capacity, int64_t* values, hipStream_t s);
hipError_t launch_dict_pool(const int64_t* values, int64_t nnz, const int64_t* offsets,
                            int64_t batch, int32_t num_tables, const void* hot,
                            int64_t hot_rows, const void* cold, int64_t cold_rows, int elt,
                            int dim, float* out, int64_t sb, int64_t st, hipStream_t s);

// interaction.hip.  pairs: the pair set, kPairStrict (i > j), kPairSelf (i >= j) or
// kPairGram (the whole F x F Gram matrix).
constexpr int kPairStrict = 0, kPairSelf = 1, kPairGram = 2;
bool interaction_bf16_supported(int F, int dim, int pairs);
bool interaction_f32_supported(int F, int dim, int pairs);
// z_bf16: Z held in bf16 (strict pairs on matrix cores, and a bf16 dZ in the backward;
// anything else returns hipErrorInvalidValue); otherwise fp32.
hipError_t launch_interaction_fwd(const void* Z, bool z_bf16, int64_t batch, int F, int dim,
                                  bool bf16, int pairs, float* R, int64_t r_stride,
                                  hipStream_t s);
hipError_t launch_interaction_bwd(const void* Z, bool z_bf16, const float* dR,
                                  int64_t dr_stride, int64_t batch, int F, int dim, bool bf16,
                                  int pairs, bool out_bf16, void* dZ, hipStream_t s);
hipError_t launch_fm_fwd(const float* Z, int64_t batch, int F, int dim, float* out,
                         hipStream_t s);
hipError_t launch_fm_bwd(const float* Z, const float* dout, int64_t batch, int F, int dim,
                         float* dZ, hipStream_t s);

// fused.hip: pooling and the dot interaction in one pass
bool embbag_interaction_supported(int num_tables, int dim, bool table_bf16, bool bf16);
hipError_t launch_embbag_interaction_fwd(const void* table, bool table_bf16, int64_t total_rows,
                                         int dim, const int64_t* row_base, int num_tables,
                                         const void* idx, bool idx64, int64_t nnz,
                                         const int64_t* offsets, int64_t batch, float* Z,
                                         bool bf16, float* R, int64_t r_stride, hipStream_t s);

// dense.hip: fully connected layers and the logistic head
int dense_wgrad_splits(int64_t M, int N, int cols, bool bf16, int64_t* k_split);
int dense_dx_splits(int64_t M, int N, int K, int64_t* k_split);
size_t dense_bwd_workspace_bytes(int64_t M, int N, int K, bool bias, bool relu, bool bf16);
hipError_t launch_dense_fwd(const float* X, int64_t xs, int64_t M, int K, const float* W,
                            const float* b, int N, bool relu, bool bf16, float* Y, int64_t ys,
                            hipStream_t s);
hipError_t launch_dense_bwd_sgd(const float* X, int64_t xs, int64_t M, int K, float* W,
                                float* b, int N, bool relu, const float* Y, int64_t ys,
                                const void* dY, bool dy_bf16, int64_t dys, bool bf16, float lr,
                                float* dX, int64_t dxs, void* workspace, hipStream_t s);
hipError_t launch_logistic_ne(const float* logits, int64_t ls, const float* labels, int64_t M,
                              float* prob, float* dlogits, int64_t dls, float* stats,
                              hipStream_t s);

}  // namespace ctr
