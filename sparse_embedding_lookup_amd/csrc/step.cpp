// step.cpp -- one training step of the sparse front end enqueued from native code: every
// call of the path, the fork and join of the unique's side stream, and optional timing
// events around the pooling kernel or the backward's first kernel, in one C call (the per-call cost of an interpreter
// would otherwise exceed the GPU time of a small batch).
//
// The step is the chain the pages describe: the batch's IDs deduplicated into contiguous
// indices ("How TensorNet Supercharges Sparse Feature Training on TensorFlow", "Core
// Optimizations"), sum-pooled lookups ("DHEN" notes, 2.1), the pairwise-dot interaction
// ("Meta DLRM", 02), and the backward that updates only the rows present in the batch
// (TensorNet page, "Synchronous Architecture").  Each call below is the public entry point
// with its own checks; nothing here computes.
#include <hip/hip_runtime.h>

#include "../../include/ctr.h"
#include "ctr_internal.h"

namespace {

int32_t invalid(const char* msg) { return ctr::set_error(CTR_ERR_INVALID_ARGUMENT, msg); }

int32_t record(void* ev, hipStream_t s) {
  if (!ev) return CTR_OK;
  const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(ev), s);
  return e == hipSuccess ? CTR_OK : ctr::set_error(CTR_ERR_HIP, hipGetErrorString(e));
}

// A timing mark (capture-aware: see ctr::record_mark).
int32_t mark(void* ev, hipStream_t s) {
  const hipError_t e = ctr::record_mark(ev, s);
  return e == hipSuccess ? CTR_OK : ctr::set_error(CTR_ERR_HIP, hipGetErrorString(e));
}

int32_t wait(hipStream_t s, void* ev) {
  const hipError_t e = hipStreamWaitEvent(s, static_cast<hipEvent_t>(ev), 0);
  return e == hipSuccess ? CTR_OK : ctr::set_error(CTR_ERR_HIP, hipGetErrorString(e));
}

#define CTR_TRY(x)                  \
  do {                              \
    const int32_t st_ = (x);        \
    if (st_ != CTR_OK) return st_;  \
  } while (0)

// The batch's unique into output set `set`, with workspace 0 (ws_unique) or 1 (ws_unique2).
int32_t unique_into(const ctr_step_t* d, int set, void* stream, int ws = 0) {
  void* wsp = ws ? d->ws_unique2 : d->ws_unique;
  size_t wsb = ws ? d->ws_unique2_bytes : d->ws_unique_bytes;
  if (d->kind == CTR_STEP_POOLED_INTERACTION)
    return ctr_unique_ids(d->indices, d->index_type, d->nnz, d->offsets, d->batch,
                          d->num_tables, d->row_base, d->total_rows, d->max_table_rows, 0,
                          d->uniq[set],
                          d->inverse[set], d->num_unique[set], d->perm[set], d->seg_offsets[set],
                          d->sorted_src[set], d->src_layout, wsp, &wsb, stream);
  return ctr_unique_ids(d->indices, d->index_type, d->nnz, nullptr, 0, 0, nullptr, 0, 0,
                        d->key_modulus, d->uniq[set], d->inverse[set], d->num_unique[set],
                        d->perm[set], d->seg_offsets[set], d->sorted_src[set], d->src_layout,
                        wsp, &wsb, stream);
}

// The stages before the unique may fork (pooling, and for the batch-matrix step the gather).
// The timing marks bracket the pooling kernel unless the descriptor puts them on the backward.
int32_t forward_part(const ctr_step_t* d, int set, hipStream_t s, void* mark_begin,
                     void* mark_end) {
  if (d->mark_stage != CTR_MARK_POOLING) mark_begin = mark_end = nullptr;
  if (d->kind == CTR_STEP_POOLED_INTERACTION) {
    const int64_t F = (int64_t)d->num_tables + 1;
    CTR_TRY(mark(mark_begin, s));
    size_t wsb = d->ws_pool_bytes;
    const size_t zsz = d->z_dtype == CTR_BF16 ? 2 : 4;      // Z[:, 1 + t, :]: past the dense row
    CTR_TRY(ctr_embbag_fwd(d->table, d->dtype, d->total_rows, d->dim, d->row_base, d->num_tables,
                           d->indices, d->index_type, d->nnz, d->offsets, d->batch,
                           static_cast<char*>(d->Z) + (size_t)d->dim * zsz, d->z_dtype,
                           F * d->dim, d->dim, d->ws_pool, &wsb, s));
    return mark(mark_end, s);
  }
  CTR_TRY(ctr_gather_rows(d->table, d->dtype, d->total_rows, d->dim, d->uniq[set],
                          d->num_unique[set], d->nnz, d->E, s));
  CTR_TRY(mark(mark_begin, s));
  size_t wsb = d->ws_pool_bytes;
  CTR_TRY(ctr_embbag_fwd(d->E, CTR_F32, d->nnz, d->dim, nullptr, 1, d->inverse[set], CTR_I32,
                         d->nnz, d->offsets, d->nnz, d->out, CTR_F32, d->dim, 0, d->ws_pool,
                         &wsb, s));
  return mark(mark_end, s);
}

// The interaction and its gradient (pooled step only).
int32_t interaction_part(const ctr_step_t* d, hipStream_t s) {
  if (d->kind != CTR_STEP_POOLED_INTERACTION) return CTR_OK;
  const int64_t F = (int64_t)d->num_tables + 1;
  CTR_TRY(ctr_dot_interaction_fwd(d->Z, d->z_dtype, d->batch, (int32_t)F, d->dim, d->compute,
                                  d->R, d->dim + F * (F - 1) / 2, s));
  return ctr_dot_interaction_bwd(d->Z, d->z_dtype, d->dR, d->dim + F * (F - 1) / 2, d->batch,
                                 (int32_t)F, d->dim, d->compute, d->grad_dtype, d->dZ, s);
}

// The backward with the SGD update of the touched rows; with mark_stage CTR_MARK_BACKWARD the
// timing marks bracket its first reduce-by-key kernel (over every sorted position).
int32_t sgd_part(const ctr_step_t* d, int set, int64_t k, hipStream_t s, void* mark_begin,
                 void* mark_end) {
  if (d->mark_stage != CTR_MARK_BACKWARD) mark_begin = mark_end = nullptr;
  const int64_t F = (int64_t)d->num_tables + 1;
  size_t wsb = d->ws_bwd_bytes;
  const bool pooled = d->kind == CTR_STEP_POOLED_INTERACTION;
  // dZ[:, 1:, :] of the pooled step (fp32 or bf16 elements), or dout
  const size_t esz = (pooled && d->grad_dtype == CTR_BF16) ? 2 : 4;
  const void* grad = pooled ? static_cast<const void*>(static_cast<const char*>(d->dZ) +
                                                       (size_t)d->dim * esz)
                            : static_cast<const void*>(d->dout);
  const int32_t gdt = pooled ? d->grad_dtype : CTR_F32;
  const int64_t sb = pooled ? F * d->dim : d->dim;
  const int64_t st = pooled ? d->dim : 0;
  const int64_t batch = pooled ? d->batch : d->nnz;
  const int32_t tables = pooled ? d->num_tables : 1;
  const bool sr = d->rounding == CTR_ROUND_STOCHASTIC;
  return ctr::embbag_bwd_sgd_marked(grad, gdt, sb, st, d->offsets, batch, tables, d->nnz,
                                    d->sorted_src[set], d->src_layout, d->num_unique[set],
                                    d->table, d->dtype,
                                    d->total_rows, d->dim, d->uniq[set], d->lr, d->rounding,
                                    sr ? ctr_sr_step_seed(d->sr_seed, k) : 0, d->row_grads,
                                    d->ws_bwd, &wsb, s, mark_begin, mark_end);
}

}  // namespace

extern "C" {

int32_t ctr_step_unique(const ctr_step_t* d, int32_t set, void* stream) {
  if (!d) return invalid("step is NULL");
  if (d->kind != CTR_STEP_POOLED_INTERACTION && d->kind != CTR_STEP_BATCH_MATRIX)
    return invalid("unknown step kind");
  if (set < 0 || set >= CTR_STEP_SETS) return invalid("set must be 0, 1 or 2");
  return unique_into(d, set, stream);
}

int32_t ctr_step_run_deep(const ctr_step_t* d, int64_t k, void* main_stream, void* side_stream0,
                          void* side_stream1, void* const* events, void* mark_begin,
                          void* mark_end) {
  if (!d) return invalid("step is NULL");
  if (d->kind != CTR_STEP_POOLED_INTERACTION && d->kind != CTR_STEP_BATCH_MATRIX)
    return invalid("unknown step kind");
  if (k < 0) return invalid("step index k < 0");
  if (d->rounding != CTR_ROUND_NEAREST && d->rounding != CTR_ROUND_STOCHASTIC)
    return invalid("unknown rounding");
  if (d->grad_dtype != CTR_F32 && d->grad_dtype != CTR_BF16) return invalid("unknown grad_dtype");
  if (!d->ws_pool) return invalid("the pooling workspace ws_pool is required");
  if (d->kind == CTR_STEP_BATCH_MATRIX)
    for (int j = 0; j < CTR_STEP_SETS; ++j)
      if (!d->inverse[j]) return invalid("the batch-matrix step pools through inverse[]");
  if (d->mark_stage != CTR_MARK_POOLING && d->mark_stage != CTR_MARK_BACKWARD)
    return invalid("unknown mark_stage");
  if (!side_stream0 || !side_stream1 || !events) return invalid("two side streams and six events are required");
  for (int i = 0; i < 6; ++i)
    if (!events[i]) return invalid("two side streams and six events are required");
  if (!d->ws_unique2) return invalid("the two-deep schedule needs the second unique workspace");
  hipStream_t s = static_cast<hipStream_t>(main_stream);
  hipStream_t side = static_cast<hipStream_t>((k & 1) ? side_stream1 : side_stream0);
  void* const* udone = events;            // udone[j]: the unique that filled set j is done
  void* const* bdone = events + 3;        // bdone[j]: the backward that read set j is done
  const int cur = (int)(k % 3), ahead = (int)((k + 2) % 3);
  // Batch k trains on set k % 3: filled by the unique forked in step k - 2, or, for the first
  // two steps, by the caller on the main stream before step 0 (so that a captured sequence
  // of steps waits on nothing recorded outside it).
  CTR_TRY(forward_part(d, cur, s, mark_begin, mark_end));
  CTR_TRY(interaction_part(d, s));
  if (k >= 2) CTR_TRY(wait(s, udone[cur]));
  // Batch k + 2's unique, on the side stream of its parity, into the set the backward of
  // step k - 1 released (step 0: a set nothing has read; the record only forks the stream).
  if (k == 0) CTR_TRY(record(bdone[ahead], s));
  CTR_TRY(wait(side, bdone[ahead]));
  // two uniques can run at once, one per side stream: each stream has its own workspace
  CTR_TRY(unique_into(d, ahead, side, (int)(k & 1)));
  CTR_TRY(record(udone[ahead], side));
  CTR_TRY(sgd_part(d, cur, k, s, mark_begin, mark_end));
  return record(bdone[cur], s);
}

int32_t ctr_step_run(const ctr_step_t* d, int64_t k, int32_t schedule, void* main_stream,
                     void* side_stream, void* fork_event, void* join_event, void* mark_begin,
                     void* mark_end) {
  if (!d) return invalid("step is NULL");
  if (d->kind != CTR_STEP_POOLED_INTERACTION && d->kind != CTR_STEP_BATCH_MATRIX)
    return invalid("unknown step kind");
  if (k < 0) return invalid("step index k < 0");
  if (d->rounding != CTR_ROUND_NEAREST && d->rounding != CTR_ROUND_STOCHASTIC)
    return invalid("unknown rounding");
  if (d->grad_dtype != CTR_F32 && d->grad_dtype != CTR_BF16) return invalid("unknown grad_dtype");
  if (!d->ws_pool) return invalid("the pooling workspace ws_pool is required");
  if (d->kind == CTR_STEP_BATCH_MATRIX)
    for (int j = 0; j < CTR_STEP_SETS; ++j)
      if (!d->inverse[j]) return invalid("the batch-matrix step pools through inverse[]");
  if (d->mark_stage != CTR_MARK_POOLING && d->mark_stage != CTR_MARK_BACKWARD)
    return invalid("unknown mark_stage");
  if (schedule < CTR_SCHEDULE_SERIAL || schedule > CTR_SCHEDULE_PIPELINED_OVERLAP)
    return invalid("unknown schedule");
  if (side_stream && (!fork_event || !join_event))
    return invalid("a side stream needs fork and join events");
  if (schedule != CTR_SCHEDULE_SERIAL && !side_stream)
    return invalid("the pipelined schedule needs a side stream");
  hipStream_t s = static_cast<hipStream_t>(main_stream);
  hipStream_t side = static_cast<hipStream_t>(side_stream);

  if (schedule == CTR_SCHEDULE_SERIAL) {
    // the batch's own unique first (beside the pooling and the interaction when the pooled
    // step has a side stream), into set 0
    const bool fork = side && d->kind == CTR_STEP_POOLED_INTERACTION;
    if (fork) {
      CTR_TRY(record(fork_event, s));
      CTR_TRY(wait(side, fork_event));
      CTR_TRY(unique_into(d, 0, side));
      CTR_TRY(record(join_event, side));
    } else {
      CTR_TRY(unique_into(d, 0, s));
    }
    CTR_TRY(forward_part(d, 0, s, mark_begin, mark_end));
    CTR_TRY(interaction_part(d, s));
    if (fork) CTR_TRY(wait(s, join_event));
    return sgd_part(d, 0, k, s, mark_begin, mark_end);
  }
  const int cur = (int)(k & 1), nxt = cur ^ 1;
  if (schedule == CTR_SCHEDULE_PIPELINED_OVERLAP) {
    // Only what the data needs: the backward of batch k waits for batch k's unique (recorded
    // as join_event in step k-1), and batch k+1's unique waits for the backward of step k-1
    // (fork_event), which released that set.  Host order matters: main's wait is enqueued
    // before this step re-records join_event.
    CTR_TRY(forward_part(d, cur, s, mark_begin, mark_end));
    CTR_TRY(interaction_part(d, s));
    if (k > 0) CTR_TRY(wait(s, join_event));
    else CTR_TRY(record(fork_event, s));
    CTR_TRY(wait(side, fork_event));
    CTR_TRY(unique_into(d, nxt, side));
    CTR_TRY(record(join_event, side));
    CTR_TRY(sgd_part(d, cur, k, s, mark_begin, mark_end));
    return record(fork_event, s);
  }
  // pipelined: batch k uses set k % 2 (filled during step k-1, or by ctr_step_unique before
  // the first step); batch k+1's unique fills the other set on the side stream, forked after
  // the pooling kernel (or when the step starts) and joined before the step ends
  const bool early = schedule == CTR_SCHEDULE_PIPELINED_EARLY;
  if (!early) CTR_TRY(forward_part(d, cur, s, mark_begin, mark_end));
  CTR_TRY(record(fork_event, s));
  CTR_TRY(wait(side, fork_event));
  CTR_TRY(unique_into(d, nxt, side));
  CTR_TRY(record(join_event, side));
  if (early) CTR_TRY(forward_part(d, cur, s, mark_begin, mark_end));
  CTR_TRY(interaction_part(d, s));
  CTR_TRY(sgd_part(d, cur, k, s, mark_begin, mark_end));
  return wait(s, join_event);
}

}  // extern "C"
