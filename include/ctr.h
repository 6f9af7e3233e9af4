/*
 * ctr.h -- C ABI of libctr, the MI355X (gfx950) sparse front end of a CTR ranking model.
 *
 * The path: batch ID deduplication (sort, unique, inverse map), a fetch of the batch's
 * rows into a batch-sized matrix, sum-pooled embedding bags, the pairwise-dot interaction
 * of the pooled vectors with the dense vector, and backward: the interaction gradient, the
 * per-row gradient sum and a sparse SGD update of the touched rows only.
 *
 * Sources (web pages, by title and section):
 *   [TN]   "How TensorNet Supercharges Sparse Feature Training on TensorFlow",
 *          "Core Optimizations" (collect the batch's IDs, sort them, give each a contiguous
 *          index, fetch rows into a matrix sized to the batch) and "Synchronous
 *          Architecture" (only the features present in the batch are synchronized).
 *   [DHEN] "DHEN" notes (calwoo.github.io), 2.1 "Feature Processing Layer" (a trainable
 *          d-dim vector per categorical term, dense features to one d-dim vector, all
 *          slots concatenated) and 3.1 "AdvancedDLRM" with Solution 2 (all pairwise inner
 *          products, C(m,2) of them, concatenated with the dense features).
 *   [DLRM] "Meta DLRM" (upskillscore.com), 02 "Arquitetura": the interaction is the dot
 *          product between all pairs of embedding vectors and the processed dense features.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is DEVICE memory unless marked "host".  The caller owns all
 *     buffers; the library never allocates, frees or synchronizes.  Each call only enqueues
 *     work on `stream` (a hipStream_t; NULL is the null stream) and returns.
 *   - Arguments are checked on the host before any launch; a bad argument returns a status
 *     without touching the device: CTR_ERR_INVALID_ARGUMENT (null required pointer, negative
 *     or too large size, F < 2, stride smaller than the row), CTR_ERR_UNSUPPORTED (pointer
 *     not 16-byte aligned, dim not a multiple of the 16-byte vector, dim or F beyond the
 *     kernel's limits), CTR_ERR_WORKSPACE_TOO_SMALL.  A launch failure returns CTR_ERR_HIP.
 *     ctr_last_error_message() gives a thread-local text of the last failure.
 *   - Sizes that index elements must be < 2^31 (n, nnz, number of bags).
 *   - Data preconditions (0 <= index < rows of its table, offsets non-decreasing from 0 to
 *     nnz) are not checked on the hot path; ctr_validate_csr checks them.  Kernels clamp
 *     every device-side index so that bad data gives bad numbers (NaN rows for out-of-range
 *     lookups), never an out-of-bounds access.
 *   - Device counts (num_unique) stay on the device; consumers read them there and launch
 *     for the capacity.
 *   - Calls that take `workspace` use a two-call query: with workspace == NULL the call only
 *     stores the required byte count in *workspace_bytes and returns CTR_OK.  A workspace
 *     must be 16-byte aligned (CTR_ERR_UNSUPPORTED otherwise).
 *   - Tables: all tables of a model live in ONE row-major allocation [total_rows, dim] of
 *     fp32, bf16 or fp16 (16-byte aligned); table t owns rows [row_base[t], row_base[t+1]).
 *     Reads widen the stored values to fp32 exactly.
 *     Bags are CSR, table-major: bag (t, b) spans indices[offsets[t*batch+b] ..
 *     offsets[t*batch+b+1]).
 */
#ifndef CTR_H
#define CTR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CTR_OK = 0,
  CTR_ERR_INVALID_ARGUMENT = 1,
  CTR_ERR_UNSUPPORTED = 2,
  CTR_ERR_WORKSPACE_TOO_SMALL = 3,
  CTR_ERR_HIP = 4
} ctr_status_t;

/* Element types.  Tables: CTR_F32, CTR_BF16 or CTR_F16 (IEEE binary16, "DHEN" notes 6.4: FP16
 * embeddings); gradients, interaction operands and dZ: CTR_F32 or CTR_BF16. */
typedef enum { CTR_F32 = 0, CTR_BF16 = 1, CTR_F16 = 2 } ctr_dtype_t;
typedef enum { CTR_I32 = 0, CTR_I64 = 1 } ctr_index_t;
/* Layout of sorted_src, one entry per sorted position (ctr_unique_ids writes it, the
 * backward reads it):
 *   CTR_SRC_FULL  int32 quadruples (u, bag, key low word, key high word), 16-byte aligned;
 *   CTR_SRC_ROWS  int32 pairs (key, bag), 8-byte aligned: the key (a table row, below 2^31)
 *                 stands in for u as the key that groups the positions, so the pair carries
 *                 half the bytes; for the fused update without row gradients, which needs
 *                 only the rows. */
typedef enum { CTR_SRC_FULL = 0, CTR_SRC_ROWS = 1 } ctr_src_layout_t;

/* Library version (major*10000 + minor*100 + patch).  0.2.0 added src_layout (ctr_unique_ids,
 * ctr_embbag_bwd_sgd*), out_dtype (ctr_embbag_fwd) and z_dtype (ctr_dot_interaction_fwd/bwd,
 * ctr_step_t). */
int32_t ctr_version(void);

/* Text of a status code (static storage). */
const char* ctr_status_string(int32_t status);

/* Thread-local text of the last failure in this thread ("" if none). */
const char* ctr_last_error_message(void);

/*
 * ctr_unique_ids -- [TN] "Core Optimizations": collect the batch's IDs, sort them and give
 * each distinct ID a contiguous index (the virtual sparse feature).
 *
 * Key of occurrence i (a1):
 *   id   = ids[i] (int32 or int64 per id_type)
 *   r    = key_modulus > 0 ? floor_mod(id, key_modulus) : id
 *   key  = (row_base != NULL ? row_base[t] : 0) + r, where bag (t, b) holds occurrence i
 *          (offsets/batch/num_tables give the bags; offsets is required with row_base).
 * Outputs (a2), with U = number of distinct keys:
 *   uniq[u]          distinct keys ascending (signed compare), u < U          int64 [n]
 *   inverse[i]       u such that uniq[u] == key(i)                            int32 [n]
 *                    (nullable: a caller that reads sorted_src instead, as the backward of
 *                    the pooling does, can leave the map out; with bags, 32-bit keys and no
 *                    perm either, the sort then moves keys and bags only)
 *   num_unique[0]    U                                                        int32 (device)
 *   perm[p]          occurrence at sorted position p, ties in occurrence order int32 [n]
 *                    (nullable)
 *   seg_offsets[u]   first sorted position of uniq[u]; seg_offsets[U] = n      int32 [n+1]
 *                    (nullable)
 *   sorted_src[4p .. 4p+3]  (u, bag, key low word, key high word) of the occurrence at
 *                    sorted position p: int32 quadruples [n] (nullable; 16-byte aligned).
 *                    The bag is t*batch + b when offsets are given, else the occurrence
 *                    index itself; the key is uniq[u] as int64 (little-endian words).  This
 *                    is the input the backward needs, written by the same pass, so that it
 *                    reaches the gradient row and the table row of a position in one read.
 *                    With src_layout CTR_SRC_ROWS: sorted_src[2p .. 2p+1] = (key, bag), int32
 *                    pairs [n] (8-byte aligned), for keys below 2^31 (row_base with
 *                    total_rows <= 2^31 - 1, or key_modulus <= 2^31; else CTR_ERR_UNSUPPORTED).
 * Key range: with row_base the keys must lie in [0, total_rows); with only a modulus in
 * [0, key_modulus); otherwise any int64.  The sort covers only the live key bits.
 * max_table_rows (0: unknown): the row count of the largest table.  With row_base and no
 * modulus, the ids of table t must then lie in [0, min(rows_t, max_table_rows)), and the
 * sort may run per table over the bits of max_table_rows - 1 only (each table's occurrences
 * are one contiguous stretch, bags being table-major); the outputs are the same.
 * n == 0 is legal: U = 0, seg_offsets[0] = 0.
 */
int32_t ctr_unique_ids(const void* ids, int32_t id_type, int64_t n,
                       const int64_t* offsets, int64_t batch, int32_t num_tables,
                       const int64_t* row_base, int64_t total_rows, int64_t max_table_rows,
                       int64_t key_modulus,
                       int64_t* uniq, int32_t* inverse, int32_t* num_unique,
                       int32_t* perm, int32_t* seg_offsets, int32_t* sorted_src,
                       int32_t src_layout, void* workspace, size_t* workspace_bytes,
                       void* stream);

/*
 * ctr_gather_rows -- [TN] "Core Optimizations": fetch the batch's rows into the
 * batch-sized matrix.  out[u, :] = table[rows[u], :] widened to fp32, for
 * u < min(num_rows[0], capacity); rows of out at or beyond that are not written.
 * out: fp32 [capacity, dim], 16-byte aligned.
 */
int32_t ctr_gather_rows(const void* table, int32_t dtype, int64_t total_rows, int32_t dim,
                        const int64_t* rows, const int32_t* num_rows, int64_t capacity,
                        float* out, void* stream);

/*
 * ctr_embbag_fwd -- [DHEN] 2.1: one d-dim vector per sparse feature, by sum pooling.
 * For every bag (t, b), t < num_tables, b < batch:
 *   out[b*out_stride_b + t*out_stride_t + c] = sum over k in the bag of
 *       table[(row_base ? row_base[t] : 0) + indices[k], c]       (fp32 accumulation)
 * Duplicates count with multiplicity; an empty bag writes zeros.  out_dtype: CTR_F32, or
 * CTR_BF16 (the fp32 sum rounded to nearest-even once, at the store: the operand the
 * matrix-core interaction takes, in half the bytes).  out is 16-byte aligned; out_stride_* are
 * in elements and multiples of 4 (fp32) or 8 (bf16), so the pooled vectors can go straight
 * into Z[b, 1 + t, :].
 * indices: int32 or int64 [nnz]; offsets: int64 [num_tables*batch + 1].
 * A bag's rows are added in occurrence order in pieces of at most a few hundred, and the
 * pieces joined in order, except in a bag of more than 4096 occurrences: that one is summed
 * in chunks of 4096 occurrences spread over the whole GPU (each chunk over the lane groups of
 * a block, joined pairwise) and the chunks' sums are added by a fixed pairwise tree, so the
 * rounding depth grows with the logarithm of the bag's length.  Workspace (two-call query,
 * 16-byte aligned, one call at a time): the chunks' partial sums, 256 bytes when nnz <= 4096.
 */
int32_t ctr_embbag_fwd(const void* table, int32_t dtype, int64_t total_rows, int32_t dim,
                       const int64_t* row_base, int32_t num_tables,
                       const void* indices, int32_t index_type, int64_t nnz,
                       const int64_t* offsets, int64_t batch,
                       void* out, int32_t out_dtype, int64_t out_stride_b,
                       int64_t out_stride_t, void* workspace, size_t* workspace_bytes,
                       void* stream);

/*
 * ctr_embbag_bwd -- chain rule of the sum pooling, reduced per distinct row ([TN]
 * "Synchronous Architecture": only rows present in the batch receive anything).
 *   row_grads[u, c] = sum over occurrences i with inverse[i] == u of
 *                     grad[b(i)*grad_stride_b + t(i)*grad_stride_t + c]
 * where bag (t(i), b(i)) holds occurrence i.  The grouping comes from ctr_unique_ids for the
 * same occurrences: either its sorted_src quadruples (preferred: read in order; only u and
 * the bag are used here), or perm and inverse (then the bags are expanded from offsets and
 * gathered in sorted order here).
 * The sum runs in sorted order as a fixed-shape tree over chunks (deterministic, no
 * atomics).  row_grads: fp32 [nnz, dim]; rows u >= U untouched.  Workspace: two-call query.
 */
int32_t ctr_embbag_bwd(const float* grad, int64_t grad_stride_b, int64_t grad_stride_t,
                       const int64_t* offsets, int64_t batch, int32_t num_tables, int32_t dim,
                       int64_t nnz, const int32_t* perm, const int32_t* inverse,
                       const int32_t* sorted_src, const int32_t* num_unique, float* row_grads,
                       void* workspace, size_t* workspace_bytes, void* stream);

/*
 * ctr_embbag_bwd_sgd -- ctr_embbag_bwd and ctr_sparse_sgd in one pass: the moment the
 * reduce-by-key completes the gradient of distinct row u it applies
 *   table[uniq[u], :] = round(table[uniq[u], :] - lr * g[u, :])
 * with exactly the arithmetic of ctr_sparse_sgd with the same rounding and seed (so the table
 * ends bit-identical to the two-call path), without writing g to memory and reading it back.
 * Grouping and table rows come from ctr_unique_ids' sorted_src (u, bag, key); uniq serves the
 * rows of segments that span several chunks.  With src_layout CTR_SRC_ROWS the entries are
 * (row, bag) pairs: the rows key the segments and address the table, uniq is not read (may
 * be NULL), a table is required, row_grads must be NULL (there is no u to index it), and
 * total_rows must be below 2^31.  The table ends bit-identical to the CTR_SRC_FULL call.
 *   grad: grad_dtype elements, CTR_F32 or CTR_BF16 (widened exactly; the sums stay fp32),
 *         8-byte aligned for bf16, 16-byte for fp32; strides in elements as in ctr_embbag_bwd.
 *   table: dtype/total_rows/dim as in ctr_sparse_sgd (dim <= 1024), or NULL: then only
 *         row_grads is written (and required).
 *   rounding, seed: as in ctr_sparse_sgd.
 *   row_grads: fp32 [nnz, dim] or NULL (the gradients are not kept).
 * Workspace: two-call query, the same size as ctr_embbag_bwd's.
 */
int32_t ctr_embbag_bwd_sgd(const void* grad, int32_t grad_dtype, int64_t grad_stride_b,
                           int64_t grad_stride_t, const int64_t* offsets, int64_t batch,
                           int32_t num_tables, int64_t nnz, const int32_t* sorted_src,
                           int32_t src_layout, const int32_t* num_unique, void* table,
                           int32_t dtype, int64_t total_rows, int32_t dim, const int64_t* uniq,
                           float lr, int32_t rounding, uint64_t seed, float* row_grads,
                           void* workspace, size_t* workspace_bytes, void* stream);

/*
 * ctr_embbag_bwd_sgd_noalloc -- ctr_embbag_bwd_sgd without a workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results (bit for bit) as
 * ctr_embbag_bwd_sgd; sorted_src is required.  The reduce-by-key carries and the finisher's
 * ticket live in a device array of ctr_noalloc_scratch_capacity() bytes (64 MiB) that the
 * library holds on each GPU it runs on until the process ends, found once per device on the
 * first call there; the call allocates and frees nothing.  A batch whose carries need more
 * (ctr_embbag_bwd_noalloc_scratch_bytes(nnz, dim) above the capacity) returns
 * CTR_ERR_UNSUPPORTED before any launch: e.g. dim 128 with bf16 gradients holds about 3e6
 * occurrences.  Every call on a GPU shares that GPU's array, so calls that overlap on one GPU
 * (two streams, two threads) race: serialise them.
 */
int32_t ctr_embbag_bwd_sgd_noalloc(const void* grad, int32_t grad_dtype, int64_t grad_stride_b,
                                   int64_t grad_stride_t, const int64_t* offsets, int64_t batch,
                                   int32_t num_tables, int64_t nnz, const int32_t* sorted_src,
                                   int32_t src_layout, const int32_t* num_unique, void* table,
                                   int32_t dtype, int64_t total_rows, int32_t dim,
                                   const int64_t* uniq, float lr, int32_t rounding,
                                   uint64_t seed, float* row_grads, void* stream);
/* Scratch bytes ctr_embbag_bwd_sgd_noalloc needs for nnz occurrences of dim-wide rows
 * ((size_t)-1 for a bad size), and the capacity it has. */
size_t ctr_embbag_bwd_noalloc_scratch_bytes(int64_t nnz, int32_t dim);
size_t ctr_noalloc_scratch_capacity(void);

/* Rounding of an SGD store into a 16-bit (bf16 or fp16) table. */
enum { CTR_ROUND_NEAREST = 0, CTR_ROUND_STOCHASTIC = 1 };

/*
 * ctr_sparse_sgd -- update of the touched rows only ([TN] "Synchronous Architecture"):
 *   table[uniq[u], :] = round(table[uniq[u], :] - lr * row_grads[u, :])
 * for u < min(num_unique[0], capacity).  Keys must be distinct (ctr_unique_ids output), so
 * no two threads touch one row; untouched rows stay bit-identical.  Element (key, c),
 * key = uniq[u]: x = fmaf(-lr, row_grads[u, c], table[key, c]) (binary32, rounded once),
 * then stored by `rounding`:
 *   CTR_ROUND_NEAREST     x itself (fp32 table), or x rounded to bf16 / fp16 nearest-even
 *                         (fp16: beyond 65504 rounds to infinity, below 2^-14 to the
 *                         subnormal grid); `seed` is ignored.
 *   CTR_ROUND_STOCHASTIC  bf16 or fp16 table ("DHEN" notes, 6.4 "Common Optimizations":
 *                         FP16 embeddings updated with stochastic rounding):
 *       r = bits 16e .. 16e+15 (e = c mod 4) of splitmix64 from state
 *           seed ^ (key * dim + c - e)          (one generator output per 4 columns)
 *       lo = x truncated toward zero to the table type, q = that type's spacing at lo
 *       stored = lo + sign(x) * q     if r < 2^16 * (|x| - |lo|) / q
 *                lo                   otherwise
 *     i.e. round away from zero with probability (|x| - |lo|) / q, rounded up to a multiple
 *     of 2^-16 (exact for bf16, where the threshold is the low 16 bits of x's binary32
 *     pattern; fp16 drops 13 bits in its normal range, so the threshold is those bits times
 *     8), so the stored value is x in expectation over r to within q * 2^-16.  Exact values
 *     and infinities are kept, NaN stays NaN; a result beyond the type's largest finite value
 *     (fp16: |x| >= 65536, or rounding up from (65504, 65536)) is infinity.  Use a fresh seed
 *     per update (ctr_sr_step_seed).  A CTR_F32 table gives CTR_ERR_UNSUPPORTED.
 */
int32_t ctr_sparse_sgd(void* table, int32_t dtype, int64_t total_rows, int32_t dim,
                       const int64_t* uniq, const int32_t* num_unique, int64_t capacity,
                       const float* row_grads, float lr, int32_t rounding, uint64_t seed,
                       void* stream);

/* ctr_sr_step_seed -- the seed of the k-th stochastically rounded update (k >= 0) of a run
 * seeded with `base`: output k of the splitmix64 stream whose state starts at base, i.e. the
 * state after k + 1 golden-ratio increments, mixed.  ctr_step_run uses it for step k. */
uint64_t ctr_sr_step_seed(uint64_t base, int64_t k);

/*
 * ctr_dot_interaction_fwd -- [DLRM] 02, [DHEN] 3.1 and Solution 2.  Z: [batch, F, dim] (z_dtype)
 * with Z[b, 0, :] the dense vector and Z[b, 1 + t, :] the pooled vectors.
 *   R[b*r_stride + c]                      = Z[b, 0, c]            c < dim
 *   R[b*r_stride + dim + i*(i-1)/2 + j]    = <Z[b, i, :], Z[b, j, :]>   F > i > j >= 0
 * compute = CTR_F32: fp32 arithmetic.  compute = CTR_BF16: operands rounded to bf16
 * (nearest-even) on matrix cores, fp32 accumulation (dim a multiple of 16, F <= 128).
 * z_dtype: CTR_F32, or CTR_BF16 with compute = CTR_BF16 (Z held in bf16, as ctr_embbag_fwd
 * writes it with out_dtype CTR_BF16: the same operands in half the bytes; the dense
 * passthrough is then the bf16 vector, widened exactly).  Z 16-byte aligned for bf16 compute.
 */
int32_t ctr_dot_interaction_fwd(const void* Z, int32_t z_dtype, int64_t batch,
                                int32_t num_vectors, int32_t dim, int32_t compute, float* R,
                                int64_t r_stride, void* stream);

/*
 * ctr_embbag_interaction_fwd -- the pooling of ctr_embbag_fwd ([DHEN] 2.1) and the dot
 * interaction of ctr_dot_interaction_fwd ([DLRM] 02, [DHEN] 3.1 and Solution 2) in one pass.
 * Z: fp32 [batch, F, dim], contiguous, F = num_tables + 1.  Row Z[b, 0, :] (the dense vector)
 * is read; rows Z[b, 1 + t, :] are written with the pooled bags, exactly as ctr_embbag_fwd
 * with out = Z + dim, out_stride_b = F*dim, out_stride_t = dim would write them (up to the
 * order in which a bag's rows are added).  R receives what ctr_dot_interaction_fwd(Z, ...,
 * compute, R, r_stride) computes from that Z, taken from an on-chip copy of the pooled
 * vectors instead of a second read of Z; with compute = CTR_BF16 the copy is the bf16
 * (nearest-even) rounding of the fp32 pooled vectors, as the separate call rounds them.
 * table, dtype, total_rows, dim, row_base, num_tables, indices, index_type, nnz, offsets,
 * batch: as ctr_embbag_fwd, except that CTR_F16 tables are not taken (CTR_ERR_UNSUPPORTED:
 * the two separate calls cover them).  Supported: dim / (values per 16 bytes) a power of two
 * up to 32, num_tables <= 256, one sample's pooled copy within 46 KiB (bf16 compute:
 * F*(dim+8)*2 bytes, fp32: F*(dim+1)*4); compute = CTR_BF16 needs dim in {16, 32, 64, 128}
 * and F <= 128.  Other shapes return CTR_ERR_UNSUPPORTED (the two separate calls cover them).
 * Z and R must not overlap the table, indices or offsets.
 */
int32_t ctr_embbag_interaction_fwd(const void* table, int32_t dtype, int64_t total_rows,
                                   int32_t dim, const int64_t* row_base, int32_t num_tables,
                                   const void* indices, int32_t index_type, int64_t nnz,
                                   const int64_t* offsets, int64_t batch, float* Z,
                                   int32_t compute, float* R, int64_t r_stride, void* stream);

/*
 * ctr_dot_interaction_bwd -- chain rule of the above.  With dP_ij = dR[b*dr_stride + dim +
 * i*(i-1)/2 + j] for i > j:
 *   dZ[b, i, :] = sum over j != i of dP_(max(i,j), min(i,j)) * Z[b, j, :]
 *                 + (i == 0 ? dR[b*dr_stride + 0 .. dim) : 0)
 * dZ: [batch, F, dim] of dz_dtype: CTR_F32, or CTR_BF16 (nearest-even of the fp32 result;
 * needs compute = CTR_BF16).  A bf16 dZ halves the bytes the backward of the pooling re-reads
 * per occurrence; its consumer accumulates in fp32 (ctr_embbag_bwd_sgd with grad_dtype =
 * CTR_BF16).  compute as in the forward (bf16 rounds dP and Z; Z and dZ 16-byte aligned).
 * z_dtype as in the forward; a bf16 Z takes a bf16 dZ.
 */
int32_t ctr_dot_interaction_bwd(const void* Z, int32_t z_dtype, const float* dR,
                                int64_t dr_stride, int64_t batch, int32_t num_vectors,
                                int32_t dim,
                                int32_t compute, int32_t dz_dtype, void* dZ, void* stream);

/*
 * ctr_dot_interaction_self_fwd / _self_bwd -- the pair set with self-dots, [DHEN] 3.1 ("all
 * inner products for i <= j"): as ctr_dot_interaction_fwd/bwd with the pairs F > i >= j >= 0
 * in row-major lower-triangle order, P = F(F+1)/2:
 *   R[b*r_stride + dim + i*(i+1)/2 + j]   = <Z[b, i, :], Z[b, j, :]>        i >= j
 *   dZ[b, i, :] = sum over j != i of dP_(max,min) Z[b, j, :] + 2 dP_ii Z[b, i, :]
 *                 + (i == 0 ? dR[b*dr_stride + 0 .. dim) : 0)
 * Same arithmetic paths, dz_dtype, limits and errors as the strict entry points; F >= 1.
 */
int32_t ctr_dot_interaction_self_fwd(const float* Z, int64_t batch, int32_t num_vectors,
                                     int32_t dim, int32_t compute, float* R, int64_t r_stride,
                                     void* stream);
int32_t ctr_dot_interaction_self_bwd(const float* Z, const float* dR, int64_t dr_stride,
                                     int64_t batch, int32_t num_vectors, int32_t dim,
                                     int32_t compute, int32_t dz_dtype, void* dZ, void* stream);

/*
 * ctr_dot_interaction_gram_fwd / _gram_bwd -- the whole Gram matrix X X^T that a DCN-style
 * layer takes ([DHEN] 3.3, eq. (7): all pairwise interactions as an F x F matrix), both
 * triangles and the diagonal, row-major after the dense slot:
 *   R[b*r_stride + c]                 = Z[b, 0, c]                        c < dim
 *   R[b*r_stride + dim + i*F + j]     = <Z[b, i, :], Z[b, j, :]>          i, j < F
 * The dot of i > j is computed once and stored at (i, j) and (j, i), so the matrix is exactly
 * symmetric.  Backward, with dG_ij = dR[b*dr_stride + dim + i*F + j]:
 *   dZ[b, i, :] = sum over j of S_ij * Z[b, j, :] + (i == 0 ? dR[b*dr_stride + 0 .. dim) : 0)
 *   S_ij = dG_ij + dG_ji in binary32 (S_ii = 2 dG_ii); compute = CTR_BF16 rounds S and Z to
 *   bf16 for the matrix cores.
 * r_stride, dr_stride >= dim + F*F; F >= 1; otherwise as ctr_dot_interaction_fwd/bwd.
 */
int32_t ctr_dot_interaction_gram_fwd(const float* Z, int64_t batch, int32_t num_vectors,
                                     int32_t dim, int32_t compute, float* R, int64_t r_stride,
                                     void* stream);
int32_t ctr_dot_interaction_gram_bwd(const float* Z, const float* dR, int64_t dr_stride,
                                     int64_t batch, int32_t num_vectors, int32_t dim,
                                     int32_t compute, int32_t dz_dtype, void* dZ, void* stream);

/*
 * ctr_fm_interaction_fwd / _bwd -- the sum of all pair dots by the squared-norm identity,
 * [DHEN] Solution 2 (the FM trick), O(F * dim) per sample instead of O(F^2 * dim):
 *   out[b] = sum over F > i > j >= 0 of <Z[b,i,:], Z[b,j,:]>
 *          = 1/2 (||sum_i Z[b,i,:]||^2 - sum_i ||Z[b,i,:]||^2)      (fp32, the right side)
 *   dZ[b, i, :] = dout[b] * (sum_j Z[b,j,:] - Z[b,i,:])
 * Z, dZ: fp32 [batch, F, dim] contiguous; out, dout: fp32 [batch].  F >= 1.
 */
int32_t ctr_fm_interaction_fwd(const float* Z, int64_t batch, int32_t num_vectors, int32_t dim,
                               float* out, void* stream);
int32_t ctr_fm_interaction_bwd(const float* Z, const float* dout, int64_t batch,
                               int32_t num_vectors, int32_t dim, float* dZ, void* stream);

/*
 * ctr_init_tables_hash -- fills a table with the counter-based values used by the seeded
 * workloads (input preparation, not part of the method): element (r, c) of table t is
 * x = fp32(2u - 1) * fp32(1/sqrt(rows_t)) with u = (splitmix64 output from state
 * seed ^ (r*dim + c)) >> 40, times 2^-24, stored as fp32, or bf16 or fp16 nearest-even.
 * row_base_host: host int64 [num_tables + 1].
 */
int32_t ctr_init_tables_hash(void* table, int32_t dtype, int32_t dim,
                             const int64_t* row_base_host, int32_t num_tables, uint64_t seed,
                             void* stream);

/*
 * ---------------------------------------------------------------- exported dictionary
 * Inference-side lookup by raw 64-bit ID ([TN] "Inference Optimization": online inference
 * reads a pre-exported sparse embedding dictionary; no modulus), with a hot-row cache in HBM
 * in front of the full table ("Tera-scale training" review, hardware-aware framework figure:
 * GPU HBM holds the hot parameters of a hierarchical parameter server, CPU memory the warm
 * ones).
 *
 * ctr_dict_build -- the dictionary's hash table.  Key keys[i] (>= 0, distinct) maps to
 * dictionary-table row rows[i] and, when hot_slots is not NULL and hot_slots[i] >= 0, to
 * row hot_slots[i] of the HBM cache.  slots: device memory of capacity * 16 bytes (16-byte
 * aligned), capacity a power of two > n; the call clears it first.  Open addressing: the
 * home slot is splitmix64(key) mod capacity, linear probing.  status: int32[3] on the
 * device, set to the number of repeated keys (the value kept is one of theirs), negative
 * keys (skipped) and keys left without a slot (0 when n < capacity).
 */
int32_t ctr_dict_build(const int64_t* keys, const int32_t* rows, const int32_t* hot_slots,
                       int64_t n, void* slots, int64_t capacity, int32_t* status, void* stream);

/*
 * ctr_dict_lookup -- values[i] for ids[i]: the slot value ((cache slot + 1) << 32 | row,
 * cache slot + 1 = 0 when not cached), or -1 when ids[i] is not in the dictionary.
 * ids, values: int64 [n] device.
 */
int32_t ctr_dict_lookup(const int64_t* ids, int64_t n, const void* slots, int64_t capacity,
                        int64_t* values, void* stream);

/*
 * ctr_dict_embbag_fwd -- sum pooling over looked-up values (bags as in ctr_embbag_fwd):
 *   out[b*out_stride_b + t*out_stride_t + c] = sum over the bag's occurrences k of
 *     hot_rows[slot][c]   when values[k] carries cache slot `slot` < num_hot,
 *     table[row][c]       otherwise, row = low 32 bits of values[k] (< num_rows),
 *   where values[k] = -1 (not in the dictionary) adds nothing.  table: [num_rows, dim] of
 * dtype, the whole dictionary; it may be pinned host memory (hipHostMalloc, device-mapped),
 * read over the host link.  hot_rows: [num_hot, dim] of dtype in HBM, or NULL.
 */
int32_t ctr_dict_embbag_fwd(const int64_t* values, int64_t nnz, const int64_t* offsets,
                            int64_t batch, int32_t num_tables, const void* hot_rows,
                            int64_t num_hot, const void* table, int64_t num_rows, int32_t dtype,
                            int32_t dim, float* out, int64_t out_stride_b,
                            int64_t out_stride_t, void* stream);

/*
 * ctr_validate_csr -- debug check of the data preconditions: offsets[0] == 0, offsets
 * non-decreasing, offsets[last] == nnz, and 0 <= indices[k] < rows of the bag's table
 * (row_base given: rows_t = row_base[t+1] - row_base[t]; else total_rows).  Adds the number
 * of violations to bad_count[0] (int32, device; the caller zeroes it).
 */
int32_t ctr_validate_csr(const void* indices, int32_t index_type, int64_t nnz,
                         const int64_t* offsets, int64_t batch, int32_t num_tables,
                         const int64_t* row_base, int64_t total_rows, int32_t* bad_count,
                         void* stream);

/*
 * ---------------------------------------------------------------- one training step
 * ctr_step_t describes every device buffer of one training step of the front end; the
 * caller owns all of it (the library keeps no state and allocates nothing).  Two kinds:
 *
 *   CTR_STEP_POOLED_INTERACTION  tables + dense vector ("Meta DLRM" 02, "DHEN" notes 2.1):
 *     ctr_unique_ids over (indices, offsets, row_base) -> ctr_embbag_fwd into Z[:, 1:, :]
 *     -> ctr_dot_interaction_fwd (Z -> R) -> ctr_dot_interaction_bwd (dR -> dZ)
 *     -> ctr_embbag_bwd_sgd over dZ[:, 1:, :] (SGD on the touched rows, rounded by the
 *     descriptor's rounding and seed, in both kinds).
 *     Z, dZ: [batch, num_tables + 1, dim] (z_dtype, grad_dtype), Z[:, 0, :] = the dense
 *     vector (input);
 *     R, dR: fp32 [batch, dim + P], P = (num_tables + 1) * num_tables / 2.
 *   CTR_STEP_BATCH_MATRIX  one table, IDs mapped by key_modulus ([TN] "Core Optimizations"):
 *     ctr_unique_ids(indices mod key_modulus) -> ctr_gather_rows into E -> ctr_embbag_fwd over
 *     E with the inverse map (one ID per bag, offsets = 0..nnz) into out
 *     -> ctr_embbag_bwd_sgd over dout (SGD on the touched table rows).
 *     E, out, dout: fp32 [nnz, dim].
 *
 * z_dtype (pooled step): the element type of Z, CTR_F32, or CTR_BF16 with compute = CTR_BF16
 * and grad_dtype = CTR_BF16 (the pooling writes bf16 vectors, the interaction reads them; the
 * dense vector Z[:, 0, :] is then bf16 too).
 *
 * Unique outputs exist in CTR_STEP_SETS = 3 sets: the serial schedule uses set 0, the
 * pipelined schedules of ctr_step_run sets 0 and 1, ctr_step_run_deep all three (an unused
 * set may repeat set 0).  Each array has capacity nnz
 * (seg_offsets nnz + 1; sorted_src 4 int32 per position, 16-byte aligned, or 2 int32,
 * 8-byte aligned, with src_layout CTR_SRC_ROWS).  Workspaces are
 * sized by the two-call queries of ctr_unique_ids and ctr_embbag_bwd.  row_grads
 * (fp32 [nnz, dim]) is optional.
 */
enum { CTR_STEP_POOLED_INTERACTION = 0, CTR_STEP_BATCH_MATRIX = 1 };
#define CTR_STEP_SETS 3
enum {
  CTR_SCHEDULE_SERIAL = 0,
  CTR_SCHEDULE_PIPELINED = 1,
  CTR_SCHEDULE_PIPELINED_EARLY = 2,
  CTR_SCHEDULE_PIPELINED_OVERLAP = 3
};
/* Where ctr_step_run's timing marks go: around the pooling kernel, or around the backward's
 * first reduce-by-key kernel (the one over every sorted position; the carry levels after it
 * are outside the marks). */
enum { CTR_MARK_POOLING = 0, CTR_MARK_BACKWARD = 1 };

typedef struct {
  int32_t kind;
  int32_t index_type;             /* CTR_I32 or CTR_I64 */
  const void* indices;            /* [nnz] */
  int64_t nnz;
  const int64_t* offsets;         /* [num_tables*batch + 1] (pooled) or [nnz + 1] */
  int64_t batch;
  int32_t num_tables;
  int32_t dim;
  const int64_t* row_base;        /* device [num_tables + 1] (pooled step) */
  int64_t key_modulus;            /* batch-matrix step */
  void* table;
  int32_t dtype;                  /* CTR_F32 or CTR_BF16 */
  int32_t compute;                /* interaction arithmetic, CTR_F32 or CTR_BF16 */
  int64_t total_rows;
  float lr;
  void* Z;                        /* z_dtype elements */
  float* R;
  const float* dR;
  void* dZ;                       /* fp32 or bf16, see grad_dtype */
  float* E;
  float* out;
  const float* dout;
  float* row_grads;
  void* ws_unique;
  size_t ws_unique_bytes;
  void* ws_bwd;
  size_t ws_bwd_bytes;
  int64_t* uniq[CTR_STEP_SETS];
  int32_t* inverse[CTR_STEP_SETS];            /* the batch-matrix step pools through it; the
                                                 pooled step may leave it NULL (nothing in it
                                                 reads the map) */
  int32_t* num_unique[CTR_STEP_SETS];
  int32_t* perm[CTR_STEP_SETS];               /* nullable */
  int32_t* seg_offsets[CTR_STEP_SETS];        /* nullable */
  int32_t* sorted_src[CTR_STEP_SETS];
  int32_t rounding;               /* CTR_ROUND_NEAREST, or CTR_ROUND_STOCHASTIC (bf16 table):
                                     step k updates with seed ctr_sr_step_seed(sr_seed, k) */
  uint64_t sr_seed;
  int32_t grad_dtype;             /* element type of dZ: CTR_F32, or CTR_BF16 (compute must be
                                     CTR_BF16; dZ then holds bf16 [batch, F, dim]) */
  void* ws_unique2;               /* ctr_step_run_deep: the second side stream's unique */
  size_t ws_unique2_bytes;        /*   workspace (two uniques run at once) */
  int32_t mark_stage;             /* CTR_MARK_POOLING (0) or CTR_MARK_BACKWARD (1) */
  int64_t max_table_rows;         /* pooled step: rows of the largest table, or 0 (see
                                     ctr_unique_ids) */
  void* ws_pool;                  /* the pooling's workspace (ctr_embbag_fwd's query) */
  size_t ws_pool_bytes;
  int32_t src_layout;             /* sorted_src's layout, CTR_SRC_FULL or CTR_SRC_ROWS (the
                                     latter needs row_grads NULL) */
  int32_t z_dtype;                /* pooled step: Z's element type, CTR_F32 or CTR_BF16 */
} ctr_step_t;

/*
 * ctr_step_run -- enqueue training step k on main_stream (one C call for the whole chain).
 *   CTR_SCHEDULE_SERIAL     the batch's unique fills set 0 first; with a side stream the
 *                           pooled step runs it there, beside the pooling and interaction,
 *                           joined before the backward.
 *   CTR_SCHEDULE_PIPELINED  step k trains on set k % 2, which ctr_step_unique (before the
 *                           first step) or step k-1 filled; right after the pooling kernel the
 *                           next batch's unique is forked to side_stream into the other set,
 *                           and the step joins it before returning control of set k % 2.
 *                           (With one repeated batch, the next batch is the same IDs.)
 *   CTR_SCHEDULE_PIPELINED_EARLY  the same, with the next batch's unique forked when the
 *                           step starts, so that it also runs beside the pooling kernel.
 *   CTR_SCHEDULE_PIPELINED_OVERLAP  no join at the step's end: the backward of step k waits
 *                           for batch k's unique (join_event, recorded by step k-1) and batch
 *                           k+1's unique waits for the backward of step k-1 (fork_event,
 *                           recorded at the end of each step), so consecutive steps overlap.
 *                           Step 0 (k == 0) waits on nothing earlier; before reading results,
 *                           or at the end of a stream capture, make main_stream wait for
 *                           side_stream.  fork_event and join_event carry state between calls:
 *                           record nothing else into them.
 * fork_event / join_event: caller-created events (required with a side stream); mark_begin /
 * mark_end: optional events recorded on main_stream right before and after the pooling
 * kernel, or, with step->mark_stage == CTR_MARK_BACKWARD, the backward's first reduce-by-key
 * kernel.  Under stream capture (graph building) the marks become event-record nodes of the
 * graph, so that each replay leaves them timed.  Returns the first failing call's status;
 * the calls before it stay enqueued.
 */
int32_t ctr_step_run(const ctr_step_t* step, int64_t k, int32_t schedule, void* main_stream,
                     void* side_stream, void* fork_event, void* join_event, void* mark_begin,
                     void* mark_end);

/* ctr_step_unique -- the unique of the step's batch into set 0, 1 or 2 on `stream` (primes
 * the pipelined schedules). */
int32_t ctr_step_unique(const ctr_step_t* step, int32_t set, void* stream);

/*
 * ctr_step_run_deep -- the overlapped schedule two batches deep.  Step k trains on set
 * k % 3 and forks batch k+2's unique into set (k+2) % 3 on side_stream(k % 2), so that two
 * uniques (each a chain of small, latency-bound kernels) are in flight beside the main
 * chain.  Only what the data needs is ordered:
 *   the backward of step k waits for the unique that filled set k % 3 (step k >= 2);
 *   batch k+2's unique waits for the backward of step k-1, which read set (k+2) % 3.
 * Before step 0, fill sets 0 and 1 with ctr_step_unique on main_stream (steps 0 and 1 wait
 * on nothing earlier, so a captured run of steps depends on nothing outside it).  events:
 * six caller-created events, carried between calls (record nothing else into them):
 * events[0..2] = unique of set j done, events[3..5] = backward that read set j done.  Before
 * reading results (or at the end of a capture) make main_stream wait for both side streams.
 * mark_begin/mark_end as in ctr_step_run.  The uniques on side_stream0 use ws_unique, those
 * on side_stream1 ws_unique2 (both sized by ctr_unique_ids' query).
 */
int32_t ctr_step_run_deep(const ctr_step_t* step, int64_t k, void* main_stream,
                          void* side_stream0, void* side_stream1, void* const* events,
                          void* mark_begin, void* mark_end);

/*
 * ---------------------------------------------------------------- dense layers and head
 * The layers on either side of the interaction ([DLRM] 02 "Arquitetura": the continuous
 * features pass through a bottom MLP whose output is the dense vector z_0; the interaction
 * output R passes through a top MLP and a sigmoid that gives the click probability; 05: the
 * public ads data has 13 continuous features, the bottom MLP's input width) and the loss
 * ([DHEN] 7.1 "Setup": normalized entropy; Solution 17: the stable cross-entropy form).
 *
 * ctr_dense_fwd -- one fully connected layer on the matrix cores:
 *   Y[m, n] = act(sum_k X[m, k] W[n, k] + b[n]),  m < M, n < N, k < K,
 * act = max(., 0) if relu else the identity.  X: fp32 rows of stride x_stride (>= K);
 * W: fp32 [N, K] contiguous; b: fp32 [N] or NULL (no bias); Y: fp32 rows of stride y_stride
 * (>= N; e.g. Z[:, 0, :] of the interaction input with y_stride = F * dim).
 * compute: CTR_F32 (fp32 products and sums) or CTR_BF16 (X and W rounded to bf16
 * nearest-even, fp32 accumulation).  1 <= K, N <= 65536; M * N, M * K and N * (K + 1) below
 * 2^31.  Y must not overlap X, W or b.  M = 0 is a no-op.
 */
int32_t ctr_dense_fwd(const float* X, int64_t x_stride, int64_t M, int32_t K, const float* W,
                      const float* b, int32_t N, int32_t relu, int32_t compute, float* Y,
                      int64_t y_stride, void* stream);

/*
 * ctr_dense_bwd_sgd -- the layer's backward with the SGD update of its parameters fused.
 * Given dY = dL/dY (fp32, or bf16 with dy_dtype = CTR_BF16; rows of stride dy_stride):
 *   dA = dY * [Y > 0] if relu (Y: the forward's output) else dY
 *   dX = dA W          (written only if dX != NULL; uses W before the update)
 *   W  = W - lr * dA^T X,   b = b - lr * sum_m dA[m, :]   (b may be NULL)
 * Gradients are sums over the M rows.  With compute = CTR_BF16 the GEMM operands (dA, W, X)
 * are rounded to bf16 nearest-even and accumulate in fp32; the bias is the weight of a
 * constant input 1, so its gradient is the same product (rounded dA times 1).  dA is never
 * stored: it is formed from dY and Y as the GEMMs load it.  The weight-gradient reduction
 * may be split over the rows into partials summed in a fixed order: results are
 * deterministic; so may dX's reduction over the N outputs when its grid is small.
 * workspace: two-call query (dA for a ReLU layer, M * N in the compute type; the weight
 * gradient's partials, S * N * (K + 1) floats, and dX's, S' * M * K floats, when those
 * reductions are split).  dX must not overlap the other arrays.  Sizes as for
 * ctr_dense_fwd.  M = 0 is a no-op (W and b unchanged).
 */
int32_t ctr_dense_bwd_sgd(const float* X, int64_t x_stride, int64_t M, int32_t K, float* W,
                          float* b, int32_t N, int32_t relu, const float* Y, int64_t y_stride,
                          const void* dY, int32_t dy_dtype, int64_t dy_stride, int32_t compute,
                          float lr, float* dX, int64_t dx_stride, void* workspace,
                          size_t* workspace_bytes, void* stream);

/*
 * ctr_logistic_ne -- the logistic head over M >= 1 logits s[i] = logits[i * logit_stride]
 * with labels y[i] (fp32, 0 or 1; values in between are taken as given):
 *   prob[i]    = sigmoid(s[i])                          (if prob != NULL)
 *   dlogits[i * dl_stride] = (prob[i] - y[i]) / M        (if dlogits != NULL: the gradient
 *                                                         of the mean cross-entropy)
 *   stats[0] = sum_i ce_i,  ce_i = softplus(s_i) - y_i s_i   (the cross-entropy in nats)
 *   stats[1] = sum_i y_i
 *   stats[2] = NE = (stats[0] / M) / H(q),  q = stats[1] / M,
 *              H(q) = -(q ln q + (1 - q) ln(1 - q)); NaN if q is 0 or 1.
 * stats: device fp32 [3].  One block: M is a batch.
 */
int32_t ctr_logistic_ne(const float* logits, int64_t logit_stride, const float* labels,
                        int64_t M, float* prob, float* dlogits, int64_t dl_stride, float* stats,
                        void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CTR_H */
