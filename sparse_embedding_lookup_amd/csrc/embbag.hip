// embbag.hip -- row gathers on gfx950: sum-pooled embedding bags, the batch-sized matrix
// fetch, the sparse SGD row update, the counter-based table fill and a CSR checker.
//
// Layout of the work: a row of the table is `vecs` 16-byte vectors (fp32: 4 values, bf16 or
// fp16: 8 values).  A group of G lanes (G a power of two, at most 64) reads one row at a
// time; each lane loads VPL vectors per row with 128-bit loads, so a wavefront gathers 64/G
// rows per load instruction, and a group keeps kU row loads in flight.  Pooling splits a
// block's bag-aligned occurrence range evenly over its groups (bags cut at group edges are
// joined in LDS), so a long or heavy-tailed bag length does not set the kernel's tail.
//
// Pooling: "DHEN" notes, 2.1 "Feature Processing Layer" (one d-dim vector per sparse
// feature; sum pooling is the reading taken).  Fetch into the batch-sized matrix and the
// touched-rows-only update: "How TensorNet Supercharges Sparse Feature Training on
// TensorFlow", "Core Optimizations" and "Synchronous Architecture".
#include "ctr_internal.h"

namespace ctr {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

// Raw 16 bytes of a row (4 binary32 or 8 bfloat16 / binary16 values, TY a kElt code),
// widened only when accumulated.
template <int TY>
__device__ __forceinline__ void accumulate(float* acc, const uint4& x) {
  if constexpr (TY != kEltF32) {
    acc[0] += half_lo<TY>(x.x); acc[1] += half_hi<TY>(x.x);
    acc[2] += half_lo<TY>(x.y); acc[3] += half_hi<TY>(x.y);
    acc[4] += half_lo<TY>(x.z); acc[5] += half_hi<TY>(x.z);
    acc[6] += half_lo<TY>(x.w); acc[7] += half_hi<TY>(x.w);
  } else {
    acc[0] += __uint_as_float(x.x); acc[1] += __uint_as_float(x.y);
    acc[2] += __uint_as_float(x.z); acc[3] += __uint_as_float(x.w);
  }
}

// Where the pooled vectors go: element b*sb + t*st + c of `p`, fp32, or bf16 rounded to
// nearest-even once at the store (the sums stay fp32 until then); strides in elements.
struct PoolOut {
  void* p;
  int64_t sb, st;
  bool bf16;
  __device__ __forceinline__ int64_t at(int64_t b, int64_t t) const { return b * sb + t * st; }
};

// N (1, 4 or 8) consecutive values of a pooled vector at element offset `off`: one 4-, 16- or
// 32-byte fp32 store, or a 2-, 8- or 16-byte bf16 one.
template <int N>
__device__ __forceinline__ void store_pooled(const PoolOut& o, int64_t off, const float* v) {
  if (o.bf16) {
    uint16_t* q = static_cast<uint16_t*>(o.p) + off;
    if constexpr (N == 1) {
      *q = (uint16_t)f32_to_bf16_bits(v[0]);
    } else {
      uint32_t w[N / 2];
#pragma unroll
      for (int i = 0; i < N / 2; ++i)
        w[i] = f32_to_bf16_bits(v[2 * i]) | (f32_to_bf16_bits(v[2 * i + 1]) << 16);
      if constexpr (N == 4) *reinterpret_cast<uint2*>(q) = make_uint2(w[0], w[1]);
      else *reinterpret_cast<uint4*>(q) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
    float* q = static_cast<float*>(o.p) + off;
    if constexpr (N == 1) {
      *q = v[0];
    } else {
      reinterpret_cast<float4*>(q)[0] = make_float4(v[0], v[1], v[2], v[3]);
      if constexpr (N == 8) reinterpret_cast<float4*>(q)[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

constexpr int kMaxBagsPerGroup = 16;

// A bag of more than kLongBag occurrences is not pooled by the kernels below (they skip its
// rows and raise a flag in the workspace) but by the long-bag kernels further down: in fixed
// chunks of kLongChunk occurrences spread over the grid, whose partial sums a fixed pairwise
// tree then adds.  A long bag is longer than a chunk, so one chunk meets at most two long
// bags and at most one starts in it.  Without the flag the long-bag kernels return at once.
constexpr int64_t kLongBag = 4096;
constexpr int64_t kLongChunk = 4096;
constexpr int64_t kLongGrid = 1024;             // blocks of the long-bag kernels (grid-stride)
static_assert(kLongBag >= kLongChunk, "a long bag spans more than one chunk");

// A group of G lanes pools `nbg` consecutive bags: their offsets and table bases go to LDS,
// their occurrences are walked in order in chunks of kU (indices loaded cooperatively and
// broadcast by shuffles, kU row loads in flight), and a bag's sum is stored when the walk
// passes its end.  Rows of a bag are added in occurrence order.
template <typename TIdx, int TY, int G, int VPL>
__global__ __launch_bounds__(kThreads) void embbag_fwd_kernel(
    const char* __restrict__ table, int64_t total_rows, int64_t row_bytes, int vecs,
    const int64_t* __restrict__ row_base, const TIdx* __restrict__ idx, int64_t nnz,
    const int64_t* __restrict__ offsets, int64_t batch, int64_t num_bags, int nbg,
    PoolOut out, int32_t* __restrict__ long_flag) {
  constexpr int E = TY != kEltF32 ? 8 : 4;
  constexpr int kGroups = kThreads / G;
  constexpr int kU = (VPL == 1 && G <= 8) ? 16 : 8;   // rows in flight per group
  constexpr int kRegs = (kU + G - 1) / G;
  __shared__ int32_t s_off[kGroups][kMaxBagsPerGroup + 1];     // nnz < 2^31
  __shared__ int64_t s_base[kGroups][kMaxBagsPerGroup];
  const int lane = threadIdx.x & (G - 1);
  const int grp = threadIdx.x / G;
  const int lane0 = (threadIdx.x & 63) & ~(G - 1);
  const int64_t s0 = ((int64_t)blockIdx.x * kGroups + grp) * nbg;
  const int nb = (int)clamp64(num_bags - s0, 0, nbg);
  for (int j = lane; j <= nb; j += G) s_off[grp][j] = (int32_t)clamp64(offsets[s0 + j], 0, nnz);
  for (int j = lane; j < nb; j += G) s_base[grp][j] = row_base ? row_base[(s0 + j) / batch] : 0;
  __syncthreads();
  if (nb == 0) return;

  const int64_t o_beg = s_off[grp][0];
  const int64_t o_end = s_off[grp][nb] > o_beg ? s_off[grp][nb] : o_beg;
  float acc[VPL][E];
#pragma unroll
  for (int a = 0; a < VPL; ++a)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[a][e] = 0.f;
  int cur = 0;
  auto is_long = [&](int j) { return (int64_t)s_off[grp][j + 1] - s_off[grp][j] > kLongBag; };
  bool any_long = false;                       // only a range above kLongBag can hold one
  if (long_flag && o_end - o_beg > kLongBag)
    for (int j = 0; j < nb; ++j) any_long |= is_long(j);
  if (any_long && lane == 0) *long_flag = 1;
  auto flush = [&](int j) {                    // a long bag is written by its own kernels
    const int64_t s = s0 + j;
    const int64_t t = s / batch, b = s - t * batch;
    const int64_t o = out.at(b, t);
    const bool keep = !(any_long && is_long(j));
#pragma unroll
    for (int a = 0; a < VPL; ++a) {
      const int vi = a * G + lane;
      if (keep && vi < vecs) store_pooled<E>(out, o + (int64_t)vi * E, acc[a]);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[a][e] = 0.f;
    }
  };

  for (int64_t k0 = o_beg; k0 < o_end; k0 += kU) {
    if (any_long) {
      // the rows of a long bag are skipped: jump to its end
      int c = cur;
      while (c < nb - 1 && k0 >= s_off[grp][c + 1]) ++c;
      if (is_long(c)) {
        while (cur <= c) flush(cur++);
        k0 = (int64_t)s_off[grp][c + 1] - kU;  // the loop's step lands on the bag's end
        continue;
      }
    }
    TIdx iv[kRegs];
#pragma unroll
    for (int r = 0; r < kRegs; ++r) {
      const int e = r * G + lane;
      const int64_t k = k0 + e;
      iv[r] = (e < kU && k < o_end) ? idx[k] : (TIdx)0;
    }
    uint4 rv[kU][VPL];
    int bagu[kU];
    int c = cur;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t k = k0 + u;
      while (c < nb - 1 && k >= s_off[grp][c + 1]) ++c;
      bagu[u] = c;
      const int64_t id = (int64_t)__shfl(iv[u / G], lane0 + (u % G), 64);
      const int64_t key = s_base[grp][c] + id;
      const bool live = k < o_end;
      const bool ok = key >= 0 && key < total_rows;
#pragma unroll
      for (int a = 0; a < VPL; ++a) {
        const int vi = a * G + lane;
        if (live && ok && vi < vecs)
          rv[u][a] = *reinterpret_cast<const uint4*>(table + key * row_bytes + (int64_t)vi * 16);
        else if (live && !ok)
          rv[u][a] = make_uint4(0x7FC00000u, 0x7FC00000u, 0x7FC00000u, 0x7FC00000u);  // NaN
        else
          rv[u][a] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (k0 + u >= o_end) break;
      while (cur < bagu[u]) flush(cur++);
#pragma unroll
      for (int a = 0; a < VPL; ++a) accumulate<TY>(acc[a], rv[u][a]);
    }
  }
  while (cur < nb) flush(cur++);
}

// Balanced pooling: a block owns `nbb` consecutive bags (so its occurrence range starts and
// ends on bag edges) and splits that range evenly over its kGroups lane groups; a group sums
// the pieces of the bags in its share (rows in occurrence order, kU loads in flight), writes
// the bags it holds whole straight out, and leaves the pieces of bags that cross a group
// edge in LDS, where the group that holds a bag's first piece adds the following groups'
// pieces in order.  A long bag thus costs what a short one does instead of setting the
// kernel's tail.  Empty bags are written as zeros by one pass over the block's offsets.
constexpr int kMaxBagsPerBlock = 1024;
// Bags per block are picked so a lane group gets about kPoolRows occurrences, but the grid
// keeps at least kPoolMinBlocks blocks (several per CU) unless a group would then get fewer
// than kPoolMinRows occurrences (a short share leaves the kU-deep load window half empty).
// Measured on the Small, Criteo-shaped, Large and TensorNet workloads.
constexpr double kPoolRows = 128.0;
constexpr int64_t kPoolMinBlocks = 2048;
constexpr double kPoolMinRows = 20.0;

// The pooling of block blk (bags blk*nbb ..).  Only a block whose range exceeds kLongBag can
// hold a long bag; there every wave checks all the block's bags (a vote, no barrier).
// SKIP = false (embbag_fwd_balanced_kernel): a block that holds a long bag raises the flag and
// pools nothing, leaving all its bags to long_bag_kernel; the others run the plain loop.
// SKIP = true (long_bag_kernel): only such a block is pooled, by a loop that skips the long
// bags' rows (the chunked kernels pool those).  Keeping the skipping loop out of the fast
// kernel keeps that kernel's code as it was: the checks cost Large's pooling about 3 %.
template <typename TIdx, int TY, int G, int VPL, bool SKIP>
__device__ __forceinline__ void pool_block(
    int64_t blk, const char* __restrict__ table, int64_t total_rows, int64_t row_bytes,
    int vecs, const int64_t* __restrict__ row_base, const TIdx* __restrict__ idx, int64_t nnz,
    const int64_t* __restrict__ offsets, int64_t batch, int64_t num_bags, int nbb,
    PoolOut out, int32_t* __restrict__ long_flag) {
  constexpr int E = TY != kEltF32 ? 8 : 4;
  constexpr int kGroups = kThreads / G;
  constexpr int kU = (VPL == 1 && G <= 8) ? 16 : 8;   // rows in flight per group
  constexpr int kRegs = (kU + G - 1) / G;
  constexpr int kW = G * VPL * E;                     // floats of one row piece
  __shared__ int32_t s_off[kMaxBagsPerBlock + 1];     // nnz < 2^31
  __shared__ int64_t s_base[kMaxBagsPerBlock];
  __shared__ float s_first[kGroups][kW];              // piece that began before the share
  __shared__ float s_last[kGroups][kW];               // piece that continues past the share
  __shared__ int32_t s_fbag[kGroups], s_fcont[kGroups], s_lbag[kGroups];
  const int lane = threadIdx.x & (G - 1);
  const int grp = threadIdx.x / G;
  const int lane0 = (threadIdx.x & 63) & ~(G - 1);
  const int64_t s0 = blk * nbb;
  const int nb = (int)clamp64(num_bags - s0, 0, nbb);
  for (int j = threadIdx.x; j <= nb; j += kThreads) s_off[j] = (int32_t)clamp64(offsets[s0 + j], 0, nnz);
  for (int j = threadIdx.x; j < nb; j += kThreads) s_base[j] = row_base ? row_base[(s0 + j) / batch] : 0;
  __syncthreads();
  if (nb == 0) return;
  auto base_of = [&](int c) -> int64_t { return s_base[c]; };
  auto out_row = [&](int c) -> int64_t {
    const int64_t sg = s0 + c;
    const int64_t t = sg / batch, b = sg - t * batch;
    return out.at(b, t);
  };
  auto store = [&](int64_t o, const float (&acc)[VPL][E]) {
#pragma unroll
    for (int a = 0; a < VPL; ++a) {
      const int vi = a * G + lane;
      if (vi < vecs) store_pooled<E>(out, o + (int64_t)vi * E, acc[a]);
    }
  };
  auto to_lds = [&](float* dst, const float (&acc)[VPL][E]) {
#pragma unroll
    for (int a = 0; a < VPL; ++a)
#pragma unroll
      for (int e = 0; e < E; ++e) dst[(a * G + lane) * E + e] = acc[a][e];
  };

  const int64_t o_beg = s_off[0];
  const int64_t range = (int64_t)s_off[nb] - o_beg;
  const int64_t share = (range + kGroups - 1) / kGroups;
  const int64_t q0 = o_beg + (int64_t)grp * share;
  const int64_t q1 = q0 + share < o_beg + range ? q0 + share : o_beg + range;
  int32_t fbag = -1, fcont = 0, lbag = -1;
  auto is_long = [&](int c) { return (int64_t)s_off[c + 1] - s_off[c] > kLongBag; };
  bool any_long = false;
  if (long_flag && range > kLongBag) {
    bool mine = false;
    for (int j = threadIdx.x & 63; j < nb; j += 64) mine |= is_long(j);
    any_long = __any(mine);
  }
  if constexpr (!SKIP) {
    if (any_long) {                            // the same in every wave
      if (threadIdx.x == 0) *long_flag = 1;
      return;
    }
  } else {
    if (!any_long) return;
  }
  constexpr bool kHasLong = SKIP;
  if (q0 < q1) {
    // bag of the share's first occurrence: last c with s_off[c] <= q0 (binary search)
    int c = 0, hi = nb - 1;
    while (c < hi) {
      const int mid = (c + hi + 1) >> 1;
      if ((int64_t)s_off[mid] <= q0) c = mid; else hi = mid - 1;
    }
    bool piece_at_start = q0 == s_off[c];
    float acc[VPL][E];
#pragma unroll
    for (int a = 0; a < VPL; ++a)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[a][e] = 0.f;
    auto close_piece = [&](bool bag_ends_here) {
      if (kHasLong && is_long(c)) {            // pooled by the long-bag kernels
      } else if (piece_at_start && bag_ends_here) {
        store(out_row(c), acc);
      } else if (!piece_at_start) {            // began before this share
        fbag = c;
        fcont = bag_ends_here ? 0 : 1;
        to_lds(s_first[grp], acc);
      } else {                                 // began here, continues past the share
        lbag = c;
        to_lds(s_last[grp], acc);
      }
#pragma unroll
      for (int a = 0; a < VPL; ++a)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[a][e] = 0.f;
    };
    for (int64_t k0 = q0; k0 < q1; k0 += kU) {
      if (kHasLong && is_long(c)) {
        // the rows of a long bag are skipped: close its (empty) piece, jump to its end
        close_piece(false);
        const int64_t e = (int64_t)s_off[c + 1];
        if (e >= q1) {
          k0 = q1;
          break;
        }
        while (c < nb - 1 && e >= s_off[c + 1]) ++c;
        piece_at_start = true;                 // e is where bag c begins
        k0 = e - kU;                           // the loop's step lands on e
        continue;
      }
      TIdx iv[kRegs];
#pragma unroll
      for (int r = 0; r < kRegs; ++r) {
        const int e = r * G + lane;
        const int64_t k = k0 + e;
        iv[r] = (e < kU && k < q1) ? idx[k] : (TIdx)0;
      }
      uint4 rv[kU][VPL];
      int bagu[kU];
      int cc = c;
      // (an explicit count: without it these loops stay rolled for G <= 8, and the row
      // registers they index go to scratch memory, one load at a time)
#pragma unroll kU
      for (int u = 0; u < kU; ++u) {
        const int64_t k = k0 + u;
        while (cc < nb - 1 && k >= s_off[cc + 1]) ++cc;
        bagu[u] = cc;
        const int64_t id = (int64_t)__shfl(iv[u / G], lane0 + (u % G), 64);
        const int64_t key = base_of(cc) + id;
        const bool live = k < q1;
        const bool ok = key >= 0 && key < total_rows;
#pragma unroll
        for (int a = 0; a < VPL; ++a) {
          const int vi = a * G + lane;
          if (live && ok && vi < vecs)
            rv[u][a] = *reinterpret_cast<const uint4*>(table + key * row_bytes + (int64_t)vi * 16);
          else if (live && !ok)
            rv[u][a] = make_uint4(0x7FC00000u, 0x7FC00000u, 0x7FC00000u, 0x7FC00000u);  // NaN
          else
            rv[u][a] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
#pragma unroll kU
      for (int u = 0; u < kU; ++u) {
        if (k0 + u >= q1) break;
        if (bagu[u] != c) {                    // the piece of bag c ended at this occurrence
          close_piece(true);
          c = bagu[u];
          piece_at_start = true;               // a later bag begins inside the share
        }
#pragma unroll
        for (int a = 0; a < VPL; ++a) accumulate<TY>(acc[a], rv[u][a]);
      }
    }
    close_piece(q1 == s_off[c + 1]);
  }
  if (lane == 0) {
    s_fbag[grp] = fbag;
    s_fcont[grp] = fcont;
    s_lbag[grp] = lbag;
  }
  __syncthreads();
  // a bag that crosses share edges: its first piece's group adds the next groups' pieces
  if (s_lbag[grp] != -1) {
    const int c = s_lbag[grp];
    float acc[VPL][E];
#pragma unroll
    for (int a = 0; a < VPL; ++a)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[a][e] = s_last[grp][(a * G + lane) * E + e];
    for (int j = grp + 1; j < kGroups && s_fbag[j] == c; ++j) {
#pragma unroll
      for (int a = 0; a < VPL; ++a)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[a][e] += s_first[j][(a * G + lane) * E + e];
      if (!s_fcont[j]) break;
    }
    store(out_row(c), acc);
  }
  // empty bags
  for (int j = threadIdx.x; j < nb; j += kThreads) {
    if (s_off[j] == s_off[j + 1]) {
      const int64_t o = out_row(j);
      const float zero[4] = {0.f, 0.f, 0.f, 0.f};
      for (int c2 = 0; c2 < vecs * E; c2 += 4) store_pooled<4>(out, o + c2, zero);
    }
  }
}

template <typename TIdx, int TY, int G, int VPL>
__global__ __launch_bounds__(kThreads) void embbag_fwd_balanced_kernel(
    const char* __restrict__ table, int64_t total_rows, int64_t row_bytes, int vecs,
    const int64_t* __restrict__ row_base, const TIdx* __restrict__ idx, int64_t nnz,
    const int64_t* __restrict__ offsets, int64_t batch, int64_t num_bags, int nbb,
    PoolOut out, int32_t* __restrict__ long_flag) {
  pool_block<TIdx, TY, G, VPL, false>(blockIdx.x, table, total_rows, row_bytes, vecs, row_base,
                                      idx, nnz, offsets, batch, num_bags, nbb, out, long_flag);
}

// ----------------------------------------------------------------------------- long bags
// The last bag j with offsets[j] <= p, j < num_bags (binary search; with non-decreasing
// offsets, offsets[0] <= p < offsets[num_bags], it is the bag that holds occurrence p).
__device__ __forceinline__ int64_t bag_at(const int64_t* __restrict__ offsets,
                                          int64_t num_bags, int64_t p) {
  int64_t lo = 0, hi = num_bags;
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) >> 1;
    if (offsets[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

// long_bag_kernel, first (balanced pooling only, nbb > 0): the blocks of the balanced kernel
// that hold a long bag, pooled by pool_block<SKIP = true>.  Then the chunks: chunk
// k = occurrences [k C, (k + 1) C), C = kLongChunk, one block each.  For each long bag
// the chunk meets (at most two), the block sums the bag's rows inside the chunk: the piece is
// split evenly over the lane groups, each adding its share in occurrence order with kU loads
// in flight, and the groups' sums are joined by a pairwise tree in LDS.  The sum goes to
// partial slot 2k (the bag holding the chunk's first occurrence) or 2k + 1 (a long bag that
// starts later in the chunk); starts[k] is the long bag that starts in chunk k, or -1.
template <typename TIdx, int TY, int G, int VPL>
__global__ __launch_bounds__(kThreads) void long_bag_kernel(
    const char* __restrict__ table, int64_t total_rows, int64_t row_bytes, int vecs,
    const int64_t* __restrict__ row_base, const TIdx* __restrict__ idx, int64_t nnz,
    const int64_t* __restrict__ offsets, int64_t batch, int64_t num_bags, int nbb,
    PoolOut out, int32_t* __restrict__ long_flag,
    int64_t* __restrict__ starts, float* __restrict__ partials) {
  constexpr int E = TY != kEltF32 ? 8 : 4;
  constexpr int kGroups = kThreads / G;
  constexpr int kU = (VPL == 1 && G <= 8) ? 16 : 8;
  constexpr int kRegs = (kU + G - 1) / G;
  constexpr int kW = G * VPL * E;
  __shared__ float s_sum[kGroups][kW];
  __shared__ int64_t s_long[2];
  const int64_t chunks = (nnz + kLongChunk - 1) / kLongChunk;
  if (*long_flag == 0) {                       // no long bag in this call
    for (int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x; k < chunks;
         k += (int64_t)gridDim.x * kThreads)
      starts[k] = -1;
    return;
  }
  if constexpr (VPL == 1) {
    if (nbb > 0) {
      const int64_t nblocks = (num_bags + nbb - 1) / nbb;
      for (int64_t blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
        __syncthreads();                       // the previous block is done with the LDS
        pool_block<TIdx, TY, G, VPL, true>(blk, table, total_rows, row_bytes, vecs, row_base,
                                           idx, nnz, offsets, batch, num_bags, nbb, out,
                                           long_flag);
      }
    }
  }
  const int lane = threadIdx.x & (G - 1);
  const int grp = threadIdx.x / G;
  const int lane0 = (threadIdx.x & 63) & ~(G - 1);
  for (int64_t k = blockIdx.x; k < chunks; k += gridDim.x) {
  const int64_t c0 = k * kLongChunk;
  const int64_t c1 = c0 + kLongChunk < nnz ? c0 + kLongChunk : nnz;
  const int dim = vecs * E;
  auto off = [&](int64_t j) { return clamp64(offsets[j], 0, nnz); };
  __syncthreads();                             // the previous chunk is done with s_long
  if (threadIdx.x == 0) s_long[0] = s_long[1] = -1;
  __syncthreads();
  // the bags meeting the chunk, from the one holding c0 to the one holding c1 - 1
  const int64_t jf = bag_at(offsets, num_bags, c0);
  const int64_t jl = bag_at(offsets, num_bags, c1 - 1);
  for (int64_t j = jf + threadIdx.x; j <= jl; j += kThreads) {
    const int64_t b0 = off(j), b1 = off(j + 1);
    if (b1 - b0 > kLongBag) s_long[j == jf ? 0 : 1] = j;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t a = s_long[0];
    starts[k] = (a >= 0 && off(a) == c0) ? a : s_long[1];
  }
  for (int w = 0; w < 2; ++w) {
    const int64_t j = s_long[w];
    if (j < 0) continue;                       // the same for the whole block
    const int64_t b0 = off(j), b1 = off(j + 1);
    const int64_t p0 = b0 > c0 ? b0 : c0, p1 = b1 < c1 ? b1 : c1;
    const int64_t share = (p1 - p0 + kGroups - 1) / kGroups;
    const int64_t q0 = p0 + grp * share < p1 ? p0 + grp * share : p1;
    const int64_t q1 = q0 + share < p1 ? q0 + share : p1;
    const int64_t base = row_base ? row_base[j / batch] : 0;
    float acc[VPL][E];
#pragma unroll
    for (int a = 0; a < VPL; ++a)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[a][e] = 0.f;
    for (int64_t k0 = q0; k0 < q1; k0 += kU) {
      TIdx iv[kRegs];
#pragma unroll
      for (int r = 0; r < kRegs; ++r) {
        const int e = r * G + lane;
        const int64_t kk = k0 + e;
        iv[r] = (e < kU && kk < q1) ? idx[kk] : (TIdx)0;
      }
      uint4 rv[kU][VPL];
#pragma unroll kU
      for (int u = 0; u < kU; ++u) {
        const int64_t key = base + (int64_t)__shfl(iv[u / G], lane0 + (u % G), 64);
        const bool live = k0 + u < q1;
        const bool ok = key >= 0 && key < total_rows;
#pragma unroll
        for (int a = 0; a < VPL; ++a) {
          const int vi = a * G + lane;
          if (live && ok && vi < vecs)
            rv[u][a] = *reinterpret_cast<const uint4*>(table + key * row_bytes + (int64_t)vi * 16);
          else if (live && !ok)
            rv[u][a] = make_uint4(0x7FC00000u, 0x7FC00000u, 0x7FC00000u, 0x7FC00000u);  // NaN
          else
            rv[u][a] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
#pragma unroll kU
      for (int u = 0; u < kU; ++u) {
        if (k0 + u >= q1) break;
#pragma unroll
        for (int a = 0; a < VPL; ++a) accumulate<TY>(acc[a], rv[u][a]);
      }
    }
#pragma unroll
    for (int a = 0; a < VPL; ++a)
#pragma unroll
      for (int e = 0; e < E; ++e) s_sum[grp][(a * G + lane) * E + e] = acc[a][e];
    __syncthreads();
    for (int h = kGroups / 2; h > 0; h >>= 1) {  // pairwise over the groups
      if (grp < h) {
#pragma unroll
        for (int a = 0; a < VPL; ++a)
#pragma unroll
          for (int e = 0; e < E; ++e)
            s_sum[grp][(a * G + lane) * E + e] += s_sum[grp + h][(a * G + lane) * E + e];
      }
      __syncthreads();
    }
    float* dst = partials + (2 * k + w) * (int64_t)dim;
    for (int c = threadIdx.x; c < dim; c += kThreads) dst[c] = s_sum[0][c];
    __syncthreads();                           // s_sum is reused by the next bag
  }
  }
}

// Long bag starts[k] (chunk k holds its first occurrence) spans chunks k .. k2: its m pieces
// sit in slots 2k + (0 if it starts at the chunk's first occurrence, else 1), 2(k + 1), ...,
// 2 k2.  One block adds them pairwise in place (level h adds piece t + h into piece t for t a
// multiple of 2h), a fixed tree of depth ceil(log2 m), and writes the bag's output row.
// The flag is lowered here for the next call: the partials kernel, its only reader, is done.
__global__ __launch_bounds__(kThreads) void long_bag_combine_kernel(
    const int64_t* __restrict__ offsets, int64_t nnz, int64_t batch, int64_t num_bags,
    int32_t* __restrict__ long_flag, const int64_t* __restrict__ starts,
    float* __restrict__ partials, int dim, PoolOut out) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *long_flag = 0;
  const int64_t chunks = (nnz + kLongChunk - 1) / kLongChunk;
  for (int64_t k = blockIdx.x; k < chunks; k += gridDim.x) {
  const int64_t j = starts[k];
  if (j < 0 || j >= num_bags) continue;        // the same for the whole block
  const int64_t c0 = k * kLongChunk;
  const int64_t b0 = clamp64(offsets[j], 0, nnz), b1 = clamp64(offsets[j + 1], 0, nnz);
  if (b1 <= b0 || b0 < c0) continue;           // (only with offsets out of order)
  const int64_t k2 = (b1 - 1) / kLongChunk;
  const int64_t m = k2 - k + 1;
  auto slot = [&](int64_t t) -> float* {
    return partials + (t == 0 ? 2 * k + (b0 > c0 ? 1 : 0) : 2 * (k + t)) * (int64_t)dim;
  };
  for (int64_t h = 1; h < m; h <<= 1) {
    const int64_t pairs = (m - 1 - h) / (2 * h) + 1;         // t = 0, 2h, ... with t + h < m
    for (int64_t q = threadIdx.x; q < pairs * dim; q += kThreads) {
      const int64_t t = (q / dim) * 2 * h;
      const int c = (int)(q - (q / dim) * dim);
      slot(t)[c] += slot(t + h)[c];
    }
    __syncthreads();
  }
  const int64_t t = j / batch, b = j - t * batch;
  const int64_t o = out.at(b, t);
  const float* r = slot(0);
  for (int c = threadIdx.x; c < dim; c += kThreads) store_pooled<1>(out, o + c, r + c);
  __syncthreads();                             // before the next bag's tree
  }
}


// E[u] = W[rows[u]] widened to fp32, u < min(num_rows, capacity).
template <int TY, int G, int VPL>
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(
    const char* __restrict__ table, int64_t total_rows, int64_t row_bytes, int vecs,
    const int64_t* __restrict__ rows, const int32_t* __restrict__ num_rows, int64_t capacity,
    float* __restrict__ out, int64_t out_stride) {
  using V = Vec<TY>;
  constexpr int E = V::kElems;
  const int lane = threadIdx.x & (G - 1);
  const int64_t u = (int64_t)blockIdx.x * (kThreads / G) + threadIdx.x / G;
  const int64_t U = clamp64((int64_t)*num_rows, 0, capacity);
  if (u >= U) return;
  const int64_t key = rows[u];
  const bool ok = key >= 0 && key < total_rows;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int vi = v * G + lane;
    if (vi >= vecs) continue;
    V x;
    if (ok) x.load(table + key * row_bytes + (int64_t)vi * 16); else x.nan();
    float4* p = reinterpret_cast<float4*>(out + u * out_stride + (int64_t)vi * E);
    p[0] = make_float4(x.v[0], x.v[1], x.v[2], x.v[3]);
    if (E == 8) p[1] = make_float4(x.v[4 % E], x.v[5 % E], x.v[6 % E], x.v[7 % E]);
  }
}

// W[uniq[u]] = round(W[uniq[u]] - lr * g[u]) for u < min(num_unique, capacity); a 16-bit
// table (bfloat16 or binary16) rounds to nearest-even, or stochastically (SR) with the
// element's random bits from `seed`.
template <int TY, bool SR, int G, int VPL>
__global__ __launch_bounds__(kThreads) void sparse_sgd_kernel(
    char* __restrict__ table, int64_t total_rows, int64_t row_bytes, int vecs,
    const int64_t* __restrict__ uniq, const int32_t* __restrict__ num_unique, int64_t capacity,
    const float* __restrict__ g, int64_t g_stride, float lr, uint64_t seed) {
  using V = Vec<TY>;
  constexpr int E = V::kElems;
  const int lane = threadIdx.x & (G - 1);
  const int64_t u = (int64_t)blockIdx.x * (kThreads / G) + threadIdx.x / G;
  const int64_t U = clamp64((int64_t)*num_unique, 0, capacity);
  if (u >= U) return;
  const int64_t key = uniq[u];
  if (key < 0 || key >= total_rows) return;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int vi = v * G + lane;
    if (vi >= vecs) continue;
    char* wp = table + key * row_bytes + (int64_t)vi * 16;
    const float4* gp = reinterpret_cast<const float4*>(g + u * g_stride + (int64_t)vi * E);
    V w;
    w.load(wp);
    float gr[E];
    {
      const float4 a = gp[0];
      gr[0] = a.x; gr[1] = a.y; gr[2] = a.z; gr[3] = a.w;
      if (E == 8) {
        const float4 c = gp[1];
        gr[4 % E] = c.x; gr[5 % E] = c.y; gr[6 % E] = c.z; gr[7 % E] = c.w;
      }
    }
    float nw[E];
#pragma unroll
    for (int e = 0; e < E; ++e) nw[e] = __builtin_fmaf(-lr, gr[e], w.v[e]);
    if constexpr (TY != kEltF32) {
      uint32_t h[E];
      uint64_t bits[2] = {0, 0};
      if (SR) {
        bits[0] = sr_bits4(seed, key, (int64_t)vi * E, vecs * E);
        bits[1] = sr_bits4(seed, key, (int64_t)vi * E + 4, vecs * E);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) h[e] = to_half<TY, SR>(nw[e], sr_take(bits[e / 4], e % 4));
      uint4 q;
      q.x = h[0] | (h[1] << 16);
      q.y = h[2] | (h[3] << 16);
      q.z = h[4 % E] | (h[5 % E] << 16);
      q.w = h[6 % E] | (h[7 % E] << 16);
      *reinterpret_cast<uint4*>(wp) = q;
    } else {
      *reinterpret_cast<float4*>(wp) = make_float4(nw[0], nw[1], nw[2], nw[3]);
    }
  }
}

// Counter-based fill: element (r, c) = fp32(2u - 1) * scale, u = top 24 bits of one
// splitmix64 output from state seed ^ (r*dim + c) (Steele, Lea, Flood, OOPSLA 2014).
__device__ __forceinline__ float hash_value(uint64_t seed, int64_t r, int64_t c, int dim,
                                            float scale) {
  const uint64_t z = splitmix64_out(seed ^ (uint64_t)(r * (int64_t)dim + c));
  const float u = (float)(uint32_t)(z >> 40) * (1.0f / 16777216.0f);
  const float sgn = 2.0f * u - 1.0f;           // exact in binary32
  return __fmul_rn(sgn, scale);
}

template <int TY>
__global__ __launch_bounds__(kThreads) void init_table_kernel(char* __restrict__ table, int dim,
                                                              int64_t row_begin, int64_t rows,
                                                              float scale, uint64_t seed) {
  constexpr int E = TY != kEltF32 ? 8 : 4;
  const int64_t vecs = dim / E;
  const int64_t total = rows * vecs;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < total; q += stride) {
    const int64_t r = row_begin + q / vecs;
    const int64_t c0 = (q % vecs) * E;
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = hash_value(seed, r, c0 + e, dim, scale);
    char* p = table + (r * dim + c0) * (TY != kEltF32 ? 2 : 4);
    if constexpr (TY != kEltF32) {
      auto h = [](float f) { return to_half<TY, false>(f, 0u); };
      uint4 w;
      w.x = h(x[0]) | (h(x[1]) << 16);
      w.y = h(x[2]) | (h(x[3]) << 16);
      w.z = h(x[4 % E]) | (h(x[5 % E]) << 16);
      w.w = h(x[6 % E]) | (h(x[7 % E]) << 16);
      *reinterpret_cast<uint4*>(p) = w;
    } else {
      *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    }
  }
}

template <typename TIdx>
__global__ __launch_bounds__(kThreads) void validate_csr_kernel(
    const TIdx* __restrict__ idx, int64_t nnz, const int64_t* __restrict__ offsets,
    int64_t batch, int32_t num_tables, const int64_t* __restrict__ row_base, int64_t total_rows,
    int32_t* __restrict__ bad) {
  const int64_t nb = (int64_t)num_tables * batch;
  const int64_t s = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  int32_t errs = 0;
  if (s == 0 && offsets[0] != 0) ++errs;
  if (s == 0 && offsets[nb] != nnz) ++errs;
  if (s < nb) {
    const int64_t a = offsets[s], e = offsets[s + 1];
    if (e < a) {
      ++errs;
    } else {
      const int64_t t = s / batch;
      const int64_t rows = row_base ? row_base[t + 1] - row_base[t] : total_rows;
      const int64_t lo = clamp64(a, 0, nnz), hi = clamp64(e, 0, nnz);
      for (int64_t k = lo; k < hi; ++k) {
        const int64_t v = (int64_t)idx[k];
        if (v < 0 || v >= rows) ++errs;
      }
    }
  }
  if (errs) atomicAdd(bad, errs);
}

}  // namespace

// ----------------------------------------------------------------------------- launchers
#define CTR_DISPATCH_G_VPL(G_, VPL_, ...)                                   \
  do {                                                                      \
    switch (G_) {                                                           \
      case 1: { constexpr int G = 1, VPL = 1; __VA_ARGS__; } break;         \
      case 2: { constexpr int G = 2, VPL = 1; __VA_ARGS__; } break;         \
      case 4: { constexpr int G = 4, VPL = 1; __VA_ARGS__; } break;         \
      case 8: { constexpr int G = 8, VPL = 1; __VA_ARGS__; } break;         \
      case 16: { constexpr int G = 16, VPL = 1; __VA_ARGS__; } break;       \
      case 32: { constexpr int G = 32, VPL = 1; __VA_ARGS__; } break;       \
      default:                                                              \
        if ((VPL_) == 1) { constexpr int G = 64, VPL = 1; __VA_ARGS__; }    \
        else if ((VPL_) == 2) { constexpr int G = 64, VPL = 2; __VA_ARGS__; } \
        else { constexpr int G = 64, VPL = 4; __VA_ARGS__; }                \
        break;                                                              \
    }                                                                       \
  } while (0)

// Runs BODY with TY the kElt code `elt` as a compile-time constant.
#define CTR_DISPATCH_ELT(elt, ...)                                          \
  do {                                                                      \
    if ((elt) == kEltF16) { constexpr int TY = kEltF16; __VA_ARGS__; }      \
    else if ((elt) == kEltBF16) { constexpr int TY = kEltBF16; __VA_ARGS__; } \
    else { constexpr int TY = kEltF32; __VA_ARGS__; }                       \
  } while (0)

// Workspace: the flag (256 bytes), starts[chunks] (int64, to a 256-byte multiple), then the
// partial rows [2 chunks][dim] (fp32).
size_t embbag_fwd_workspace_bytes(int64_t nnz, int dim) {
  const int64_t chunks = nnz > kLongBag ? (nnz + kLongChunk - 1) / kLongChunk : 0;
  return 256 + ((size_t)chunks * 8 + 255) / 256 * 256 + (size_t)chunks * 2 * (size_t)dim * 4;
}

hipError_t launch_embbag_fwd(const void* table, int elt, int64_t total_rows, int dim,
                             const int64_t* row_base, int32_t num_tables, const void* idx,
                             bool idx64, int64_t nnz, const int64_t* offsets, int64_t batch,
                             void* out, bool out_bf16, int64_t sb, int64_t st, void* workspace,
                             hipStream_t s) {
  const PoolOut po{out, sb, st, out_bf16};
  const int E = elt != kEltF32 ? 8 : 4;
  const int vecs = dim / E;
  const RowGeom rg = row_geom(vecs);
  const int64_t row_bytes = (int64_t)dim * (elt != kEltF32 ? 2 : 4);
  const int64_t num_bags = (int64_t)num_tables * batch;
  if (num_bags == 0) return hipSuccess;
  const char* tb = static_cast<const char*>(table);
  const double avg = (double)nnz / (double)num_bags;
  // the long-bag flag: only needed when a bag can be long
  int32_t* long_flag = nnz > kLongBag ? static_cast<int32_t*>(workspace) : nullptr;
#define CTR_FWD_LAUNCH(KERNEL, BLOCKS, PER)                                                    \
  do {                                                                                        \
    CTR_DISPATCH_ELT(elt, {                                                                   \
      if (idx64)                                                                              \
        KERNEL<int64_t, TY, G, VPL><<<(unsigned)(BLOCKS), kThreads, 0, s>>>(                  \
            tb, total_rows, row_bytes, vecs, row_base, (const int64_t*)idx, nnz, offsets,     \
            batch, num_bags, PER, po, long_flag);                                            \
      else                                                                                    \
        KERNEL<int32_t, TY, G, VPL><<<(unsigned)(BLOCKS), kThreads, 0, s>>>(                  \
            tb, total_rows, row_bytes, vecs, row_base, (const int32_t*)idx, nnz, offsets,     \
            batch, num_bags, PER, po, long_flag);                                            \
    });                                                                                       \
  } while (0)
  int nbb_used = 0;                               // bags per block of the balanced kernel
  CTR_DISPATCH_G_VPL(rg.G, rg.VPL, {
    constexpr int kGroups = kThreads / G;
    if (VPL == 1) {
      const double per = avg > 1.0 ? avg : 1.0;
      int64_t nbb = (int64_t)(kPoolRows * kGroups / per + 0.5);
      if (nbb > num_bags / kPoolMinBlocks) nbb = num_bags / kPoolMinBlocks;
      const int64_t floor_bags = (int64_t)ceil(kPoolMinRows * kGroups / per);
      if (nbb < floor_bags) nbb = floor_bags;
      if (nbb > kMaxBagsPerBlock) nbb = kMaxBagsPerBlock;
      if (nbb < 1) nbb = 1;
      const int64_t blocks = (num_bags + nbb - 1) / nbb;
      nbb_used = (int)nbb;
      CTR_FWD_LAUNCH(embbag_fwd_balanced_kernel, blocks, (int)nbb);
      break;
    }
    // Rows of 1 KiB and more (64 lanes, several vectors each): one group per few bags.
    // Bags per lane group: about 64 occurrences per group, but keep >= 1024 blocks in flight.
    int nbg = (int)(64.0 / (avg > 1.0 ? avg : 1.0) + 0.5);
    if (nbg > kMaxBagsPerGroup) nbg = kMaxBagsPerGroup;
    const int64_t cap = num_bags / ((int64_t)kGroups * 1024);
    if (nbg > cap) nbg = (int)cap;
    if (nbg < 1) nbg = 1;
    const int64_t per_block = (int64_t)kGroups * nbg;
    const int64_t blocks = (num_bags + per_block - 1) / per_block;
    CTR_FWD_LAUNCH(embbag_fwd_kernel, blocks, nbg);
  });
#undef CTR_FWD_LAUNCH
  if (!long_flag) return hipGetLastError();        // no bag can be long
  // long bags: chunk partials, then each bag's pairwise sum (which lowers the flag again)
  const int64_t chunks = (nnz + kLongChunk - 1) / kLongChunk;
  const unsigned lgrid = (unsigned)(chunks < kLongGrid ? chunks : kLongGrid);
  int64_t* starts = reinterpret_cast<int64_t*>(static_cast<char*>(workspace) + 256);
  float* partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + 256 +
                                             ((size_t)chunks * 8 + 255) / 256 * 256);
  CTR_DISPATCH_G_VPL(rg.G, rg.VPL, {
    CTR_DISPATCH_ELT(elt, {
      if (idx64)
        long_bag_kernel<int64_t, TY, G, VPL><<<lgrid, kThreads, 0, s>>>(
            tb, total_rows, row_bytes, vecs, row_base, (const int64_t*)idx, nnz, offsets,
            batch, num_bags, nbb_used, po, long_flag, starts, partials);
      else
        long_bag_kernel<int32_t, TY, G, VPL><<<lgrid, kThreads, 0, s>>>(
            tb, total_rows, row_bytes, vecs, row_base, (const int32_t*)idx, nnz, offsets,
            batch, num_bags, nbb_used, po, long_flag, starts, partials);
    });
  });
  long_bag_combine_kernel<<<lgrid, kThreads, 0, s>>>(offsets, nnz, batch, num_bags, long_flag,
                                                     starts, partials, dim, po);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* table, int elt, int64_t total_rows, int dim,
                              const int64_t* rows, const int32_t* num_rows, int64_t capacity,
                              float* out, hipStream_t s) {
  if (capacity == 0) return hipSuccess;
  const int E = elt != kEltF32 ? 8 : 4;
  const int vecs = dim / E;
  const RowGeom rg = row_geom(vecs);
  const int64_t row_bytes = (int64_t)dim * (elt != kEltF32 ? 2 : 4);
  const char* tb = static_cast<const char*>(table);
  CTR_DISPATCH_G_VPL(rg.G, rg.VPL, {
    const int64_t blocks = (capacity + (kThreads / G) - 1) / (kThreads / G);
    CTR_DISPATCH_ELT(elt, gather_rows_kernel<TY, G, VPL><<<(unsigned)blocks, kThreads, 0, s>>>(
                              tb, total_rows, row_bytes, vecs, rows, num_rows, capacity, out,
                              dim));
  });
  return hipGetLastError();
}

hipError_t launch_sparse_sgd(void* table, int elt, int64_t total_rows, int dim,
                             const int64_t* uniq, const int32_t* num_unique, int64_t capacity,
                             const float* g, float lr, bool stochastic, uint64_t seed,
                             hipStream_t s) {
  if (capacity == 0) return hipSuccess;
  const int E = elt != kEltF32 ? 8 : 4;
  const int vecs = dim / E;
  const RowGeom rg = row_geom(vecs);
  const int64_t row_bytes = (int64_t)dim * (elt != kEltF32 ? 2 : 4);
  char* tb = static_cast<char*>(table);
  CTR_DISPATCH_G_VPL(rg.G, rg.VPL, {
    const int64_t blocks = (capacity + (kThreads / G) - 1) / (kThreads / G);
    if (elt == kEltF16 && stochastic)
      sparse_sgd_kernel<kEltF16, true, G, VPL><<<(unsigned)blocks, kThreads, 0, s>>>(
          tb, total_rows, row_bytes, vecs, uniq, num_unique, capacity, g, dim, lr, seed);
    else if (elt == kEltF16)
      sparse_sgd_kernel<kEltF16, false, G, VPL><<<(unsigned)blocks, kThreads, 0, s>>>(
          tb, total_rows, row_bytes, vecs, uniq, num_unique, capacity, g, dim, lr, seed);
    else if (elt == kEltBF16 && stochastic)
      sparse_sgd_kernel<kEltBF16, true, G, VPL><<<(unsigned)blocks, kThreads, 0, s>>>(
          tb, total_rows, row_bytes, vecs, uniq, num_unique, capacity, g, dim, lr, seed);
    else if (elt == kEltBF16)
      sparse_sgd_kernel<kEltBF16, false, G, VPL><<<(unsigned)blocks, kThreads, 0, s>>>(
          tb, total_rows, row_bytes, vecs, uniq, num_unique, capacity, g, dim, lr, seed);
    else
      sparse_sgd_kernel<kEltF32, false, G, VPL><<<(unsigned)blocks, kThreads, 0, s>>>(
          tb, total_rows, row_bytes, vecs, uniq, num_unique, capacity, g, dim, lr, seed);
  });
  return hipGetLastError();
}

hipError_t launch_init_table(void* table, int elt, int dim, int64_t row_begin, int64_t rows,
                             float scale, uint64_t seed, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int E = elt != kEltF32 ? 8 : 4;
  const int64_t total = rows * (dim / E);
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  CTR_DISPATCH_ELT(elt, init_table_kernel<TY><<<(unsigned)blocks, kThreads, 0, s>>>(
                            static_cast<char*>(table), dim, row_begin, rows, scale, seed));
  return hipGetLastError();
}

hipError_t launch_validate_csr(const void* idx, bool idx64, int64_t nnz, const int64_t* offsets,
                               int64_t batch, int32_t num_tables, const int64_t* row_base,
                               int64_t total_rows, int32_t* bad, hipStream_t s) {
  const int64_t nb = (int64_t)num_tables * batch;
  const int64_t blocks = (nb + kThreads) / kThreads;   // at least one block for the ends
  if (idx64)
    validate_csr_kernel<int64_t><<<(unsigned)blocks, kThreads, 0, s>>>(
        (const int64_t*)idx, nnz, offsets, batch, num_tables, row_base, total_rows, bad);
  else
    validate_csr_kernel<int32_t><<<(unsigned)blocks, kThreads, 0, s>>>(
        (const int32_t*)idx, nnz, offsets, batch, num_tables, row_base, total_rows, bad);
  return hipGetLastError();
}

}  // namespace ctr
