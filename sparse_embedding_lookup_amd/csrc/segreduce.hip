// segreduce.hip -- backward of sum pooling on gfx950: per-occurrence gradients summed onto
// the batch's distinct rows ("How TensorNet Supercharges Sparse Feature Training on
// TensorFlow", "Synchronous Architecture": only rows present in the batch get anything).
//
// Input: the unique step's (u, bag, table row) per sorted position, or its (table row, bag)
// when the update needs no row gradients (the row then keys the segments), or perm (sorted
// position -> occurrence) and inverse (occurrence -> u), from which two small kernels build
// (u, bag) per sorted position first (a wave expands 64 bags by a shuffle binary search
// over their ends; then one gather in sorted order).  Then a deterministic reduce-by-key
// over the sorted sequence in fixed chunks, so that a row hit a million times costs the
// same as a million rows hit once.  A workgroup owns a chunk of S*KPS positions; each
// G-lane slot (G lanes x 16 B per row) sums KPS consecutive positions, with every
// gradient row and every table row it needs requested before it adds anything, and writes
// the segments it completes straight out (row_grads and/or the SGD update); the pieces of
// segments that cross slot edges are joined in LDS; pieces that cross the chunk edges go
// out as at most two carries per chunk.  The carries (key, row) form a sequence of the same
// kind, reduced by the same kernel, until one chunk is left: a tree of fixed shape whose
// depth is ceil(log_chunk(n)).  No atomics anywhere.
#include <mutex>
#include <type_traits>

#include "ctr_internal.h"

namespace ctr {
namespace {

constexpr int kThreads = 256;
// Positions summed by one slot (KPS): fewer positions mean fewer live registers per slot and
// more slots per chunk.  The depth sets the summation tree, so it depends only on what is
// summed, never on where the sums go: with or without the update, the same gradients give
// the same row sums bit for bit.  fp32 gradient rows (16 bytes per lane) run best at 4,
// packed bf16 rows at 6 (measured on the Small, TensorNet, Criteo-shaped and Large
// workloads; with 8-column lanes, 4 and 8 were slower on Criteo and Large too).  The
// workspace is sized for the smallest depth.
template <bool GB>
constexpr int slot_depth() { return GB ? 6 : 4; }
constexpr int kMinSlotDepth = 4;
constexpr int64_t kFoldBlocks = 256;   // a level this small may finish the tree in place

__global__ __launch_bounds__(kThreads) void bag_of_kernel(const int64_t* __restrict__ offsets,
                                                          int64_t num_bags, int64_t nnz,
                                                          int32_t* __restrict__ bag_of) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t s0 = wave * 64;
  if (s0 >= num_bags) return;
  const int64_t s = s0 + lane;
  // end of bag s0+lane (bags past the last one end at +inf)
  const int64_t my_end = s < num_bags ? clamp64(offsets[s + 1], 0, nnz) : INT64_MAX;
  const int64_t beg = clamp64(offsets[s0], 0, nnz);
  const int64_t last = s0 + 64 < num_bags ? s0 + 64 : num_bags;
  const int64_t end = clamp64(offsets[last], beg, nnz);
  for (int64_t i0 = beg; i0 < end; i0 += 64) {
    const int64_t i = i0 + lane;
    // l = number of bags among the 64 whose end is <= i, i.e. the bag that holds i
    int l = 0;
#pragma unroll
    for (int step = 32; step > 0; step >>= 1) {
      const int64_t e = __shfl(my_end, l + step - 1, 64);
      if (e <= i) l += step;
    }
    if (i < end) bag_of[i] = (int32_t)(s0 + l);
  }
}

__global__ __launch_bounds__(kThreads) void seg_src_kernel(const int32_t* __restrict__ perm,
                                                           const int32_t* __restrict__ inverse,
                                                           const int32_t* __restrict__ bag_of,
                                                           int64_t n, int4* __restrict__ src) {
  const int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (p >= n) return;
  const int32_t i = perm[p];
  int4 r = make_int4(-1, 0, -1, -1);                       // the key is not needed here
  if (i >= 0 && (int64_t)i < n) r = make_int4(inverse[i], bag_of[i], -1, -1);
  src[p] = r;
}

// Level-0 entries, one per sorted position, and the per-bag gradient rows they point at, fp32
// or bf16 (GB; widened exactly).  Offsets are in elements.  An entry is 16 bytes, (u, bag,
// table row as two words), or with ROWS 8 bytes, (table row, bag): the row then stands in for
// the distinct-row index u as the key that groups the positions (the two are in one-to-one
// order-preserving correspondence), which is all the fused update needs.
template <bool GB, bool ROWS>
struct L0SourceT {
  static constexpr bool kBf16 = GB;
  static constexpr bool kRows = ROWS;
  const void* src;
  const void* grad;
  int64_t sb, st, batch, num_bags;
  struct Entry {
    int32_t key, bag;
    int64_t row;
  };
  __device__ __forceinline__ Entry entry(int64_t p) const {
    if constexpr (ROWS) {
      const int2 e = static_cast<const int2*>(src)[p];
      return Entry{e.x, e.y, (int64_t)e.x};
    } else {
      const int4 e = static_cast<const int4*>(src)[p];
      return Entry{e.x, e.y, (int64_t)(((uint64_t)(uint32_t)e.w << 32) | (uint32_t)e.z)};
    }
  }
  __device__ __forceinline__ int32_t key(int64_t p) const {
    if constexpr (ROWS) return static_cast<const int2*>(src)[p].x;
    else return static_cast<const int4*>(src)[p].x;
  }
  // Four consecutive gradient values at element offset `off` (a multiple of 4), loaded raw
  // (8 bytes of bf16, or 16 of fp32) and widened only where they are added, so that a
  // slot's loads issue together and bf16 rows stay packed in registers until then.
  using Raw = typename std::conditional<GB, uint2, float4>::type;
  __device__ __forceinline__ Raw load_raw(int64_t off) const {
    if constexpr (GB)
      return *reinterpret_cast<const uint2*>(static_cast<const __bf16*>(grad) + off);
    else
      return *reinterpret_cast<const float4*>(static_cast<const float*>(grad) + off);
  }
  static __device__ __forceinline__ Raw zero_raw() {
    if constexpr (GB) return make_uint2(0u, 0u);
    else return make_float4(0.f, 0.f, 0.f, 0.f);
  }
  static __device__ __forceinline__ float4 widen(const Raw& r) {
    if constexpr (GB)
      return make_float4(bf16_lo(r.x), bf16_hi(r.x), bf16_lo(r.y), bf16_hi(r.y));
    else
      return r;
  }
};
using L0Source = L0SourceT<false, false>;
using L0SourceB = L0SourceT<true, false>;

struct LnSource {
  static constexpr bool kBf16 = false;
  const int32_t* keys;
  const float* rows;
  int dim;
  __device__ __forceinline__ int32_t key(int64_t p) const { return keys[p]; }
};

template <int VPL>
struct RowAcc {
  float v[VPL][4];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int a = 0; a < VPL; ++a) v[a][0] = v[a][1] = v[a][2] = v[a][3] = 0.f;
  }
};

// Key of the nearest real entry before position q in a carry sequence: a run of one key
// never holds two consecutive empty (-1) entries, so looking two back is enough.
template <bool L0, typename Src>
__device__ __forceinline__ int32_t key_before(const Src& S, int64_t q) {
  if (q <= 0) return -1;
  const int32_t k = S.key(q - 1);
  if (L0 || k != -1) return k;
  return q >= 2 ? S.key(q - 2) : -1;
}
template <bool L0, typename Src>
__device__ __forceinline__ int32_t key_after(const Src& S, int64_t q, int64_t n) {
  if (q >= n) return -1;
  const int32_t k = S.key(q);
  if (L0 || k != -1) return k;
  return q + 1 < n ? S.key(q + 1) : -1;
}

// Where a finished row gradient goes besides row_grads: nowhere (MODE 0), or straight into
// the sparse SGD update W[uniq[u]] -= lr * g[u] of an fp32 (MODE 1), bf16 or fp16 table,
// rounded to nearest-even (MODE 2 bf16, 4 fp16) or stochastically with the element's bits
// from `seed` (MODE 3 bf16, 5 fp16),
// with the same arithmetic as the stand-alone update (one fused multiply-add, then the
// rounding).
struct SgdTarget {
  char* table;
  int64_t total_rows;
  int64_t row_bytes;
  const int64_t* uniq;     // the table row of each u; null when the keys are the rows
  float lr;
  uint64_t seed;
};

// The 16-bit element type and rounding of a table MODE (2..5).
template <int MODE>
constexpr int kModeElt = MODE >= 4 ? kEltF16 : kEltBF16;
template <int MODE>
constexpr bool kModeSR = MODE == 3 || MODE == 5;

// Four 16-bit table values (columns c..c+3 of row key) after W - lr * g.
template <int MODE>
__device__ __forceinline__ uint2 half_updated(const SgdTarget& sgd, int64_t key, int c,
                                              float g0, float g1, float g2, float g3,
                                              uint2 w) {
  constexpr int TY = kModeElt<MODE>;
  constexpr bool SR = kModeSR<MODE>;
  const float n[4] = {__builtin_fmaf(-sgd.lr, g0, half_lo<TY>(w.x)),
                      __builtin_fmaf(-sgd.lr, g1, half_hi<TY>(w.x)),
                      __builtin_fmaf(-sgd.lr, g2, half_lo<TY>(w.y)),
                      __builtin_fmaf(-sgd.lr, g3, half_hi<TY>(w.y))};
  uint32_t h[4];
  uint64_t bits = 0;
  if constexpr (SR) bits = sr_bits4(sgd.seed, key, c, (int)(sgd.row_bytes >> 1));
#pragma unroll
  for (int e = 0; e < 4; ++e) h[e] = to_half<TY, SR>(n[e], sr_take(bits, e));
  return make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
}

template <int G, int VPL>
struct SegSmem {
  float first_row[kThreads / G][G * VPL * 4];
  float last_row[kThreads / G][G * VPL * 4];
  int32_t first_key[kThreads / G];
  int32_t first_cont[kThreads / G];
  int32_t last_key[kThreads / G];
  int32_t wg_first_key;
  int32_t wg_last_key;
};

// Table-row part of one lane (4 columns) and its update W <- W - lr * g: one fused
// multiply-add in fp32, then a plain store (fp32) or the 16-bit rounding of the MODE.
template <int MODE>
using WVec = typename std::conditional<(MODE >= 2), uint2, float4>::type;

template <int MODE>
__device__ __forceinline__ WVec<MODE> load_wvec(const SgdTarget& sgd, int64_t key, int c,
                                                bool ok) {
  const char* wrow = sgd.table + key * sgd.row_bytes;
  if constexpr (MODE >= 2)
    return ok ? *reinterpret_cast<const uint2*>(wrow + (int64_t)c * 2) : make_uint2(0u, 0u);
  else
    return ok ? *reinterpret_cast<const float4*>(wrow + (int64_t)c * 4)
              : make_float4(0.f, 0.f, 0.f, 0.f);
}

template <int MODE>
__device__ __forceinline__ void store_updated(const SgdTarget& sgd, int64_t key, int c,
                                              const float4& g, const WVec<MODE>& x) {
  char* wrow = sgd.table + key * sgd.row_bytes;
  if constexpr (MODE == 1) {
    *reinterpret_cast<float4*>(wrow + (int64_t)c * 4) =
        make_float4(__builtin_fmaf(-sgd.lr, g.x, x.x), __builtin_fmaf(-sgd.lr, g.y, x.y),
                    __builtin_fmaf(-sgd.lr, g.z, x.z), __builtin_fmaf(-sgd.lr, g.w, x.w));
  } else if constexpr (MODE >= 2) {
    *reinterpret_cast<uint2*>(wrow + (int64_t)c * 2) =
        half_updated<MODE>(sgd, key, c, g.x, g.y, g.z, g.w, x);
  }
}

// CW columns of a table row (4, or 8 for the bf16 gradient rows' 8-column lanes): read, and
// written back as W - lr * g with the same arithmetic and rounding as four columns at a time.
template <int MODE, int CW>
struct TRow {
  WVec<MODE> v[CW / 4];
};
template <int MODE, int CW>
__device__ __forceinline__ TRow<MODE, CW> load_trow(const SgdTarget& sgd, int64_t key, int c,
                                                    bool ok) {
  TRow<MODE, CW> r;
  if constexpr (CW == 8 && MODE >= 2) {
    const uint4 q = ok ? *reinterpret_cast<const uint4*>(sgd.table + key * sgd.row_bytes +
                                                         (int64_t)c * 2)
                       : make_uint4(0u, 0u, 0u, 0u);
    r.v[0] = make_uint2(q.x, q.y);
    r.v[1] = make_uint2(q.z, q.w);
  } else {
#pragma unroll
    for (int a = 0; a < CW / 4; ++a) r.v[a] = load_wvec<MODE>(sgd, key, c + 4 * a, ok);
  }
  return r;
}
template <int MODE, int CW>
__device__ __forceinline__ void store_trow(const SgdTarget& sgd, int64_t key, int c,
                                           const float* g, const TRow<MODE, CW>& w) {
  if constexpr (CW == 8 && MODE >= 2) {
    const uint2 lo = half_updated<MODE>(sgd, key, c, g[0], g[1], g[2], g[3], w.v[0]);
    const uint2 hi = half_updated<MODE>(sgd, key, c + 4, g[4], g[5], g[6], g[7], w.v[1]);
    *reinterpret_cast<uint4*>(sgd.table + key * sgd.row_bytes + (int64_t)c * 2) =
        make_uint4(lo.x, lo.y, hi.x, hi.y);
  } else {
#pragma unroll
    for (int a = 0; a < CW / 4; ++a)
      store_updated<MODE>(sgd, key, c + 4 * a,
                          make_float4(g[4 * a], g[4 * a + 1], g[4 * a + 2], g[4 * a + 3]),
                          w.v[a]);
  }
}

// CW gradient values of one lane: 4 (one 16-byte fp32 or 8-byte bf16 vector), or 8 bf16 in
// one 16-byte vector.
template <typename Src, int CW>
struct GVec {
  using T = typename Src::Raw;
  static __device__ __forceinline__ T load(const Src& S, int64_t off) { return S.load_raw(off); }
  static __device__ __forceinline__ T zero() { return Src::zero_raw(); }
  static __device__ __forceinline__ void widen(const T& r, float* x) {
    const float4 f = Src::widen(r);
    x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
  }
};
template <typename Src>
struct GVec<Src, 8> {
  static_assert(Src::kBf16, "8-column lanes take bf16 gradient rows");
  using T = uint4;
  static __device__ __forceinline__ T load(const Src& S, int64_t off) {
    return *reinterpret_cast<const uint4*>(static_cast<const __bf16*>(S.grad) + off);
  }
  static __device__ __forceinline__ T zero() { return make_uint4(0u, 0u, 0u, 0u); }
  static __device__ __forceinline__ void widen(const T& r, float* x) {
    x[0] = bf16_lo(r.x); x[1] = bf16_hi(r.x); x[2] = bf16_lo(r.y); x[3] = bf16_hi(r.y);
    x[4] = bf16_lo(r.z); x[5] = bf16_hi(r.z); x[6] = bf16_lo(r.w); x[7] = bf16_hi(r.w);
  }
};

// The table row a slot holds for the piece it may finish after the chunk's join.
template <int MODE, int CW>
struct PendingRow {
  int64_t key = -1;
  TRow<MODE, CW> w;
};

// Sum the slot's KPS sorted positions when one vector of CW columns per lane covers a row
// (d <= CW G): CW = 4, or 8 for bf16 gradient rows (16 bytes per lane, so a wave covers
// twice the rows and each position's bookkeeping is shared by twice the bytes).  Each sorted
// position carries (u, bag, table row), so the slot issues every
// memory access it needs in two dependent rounds: its entries, then all gradient rows
// together with the table rows of the segments it completes (and of its last piece, which
// it may complete after the chunk's join).  A position ends a piece where the next key
// differs; a piece whose key equals the key just before the slot began earlier (sorted
// keys), and one whose key equals the key just after continues later: those two go to LDS
// for the join, every other piece is complete and is written out (and applied) here.
template <int G, int CW, int MODE, int KPS, typename Src>
__device__ __forceinline__ void slot_prefetched(const Src& S, int64_t q0, int64_t q1,
                                                int64_t n, int dim, int64_t capacity,
                                                float* __restrict__ row_grads,
                                                const SgdTarget& sgd, SegSmem<G, CW / 4>& sm,
                                                int slot, int lane, int32_t& fkey, int32_t& fcont,
                                                int32_t& lkey, PendingRow<MODE, CW>& pend) {
  using GV = GVec<Src, CW>;
  constexpr int kRegs = (KPS + G - 1) / G;
  const int lane0 = (threadIdx.x & 63) & ~(G - 1);
  const int len = (int)(q1 - q0);
  const int c = lane * CW;
  const bool col_ok = c < dim;
  // the lane's CW sums into LDS (the join's first / last pieces)
  auto to_lds = [&](float* row, const float* v) {
#pragma unroll
    for (int a = 0; a < CW / 4; ++a)
      *reinterpret_cast<float4*>(row + c + 4 * a) =
          make_float4(v[4 * a], v[4 * a + 1], v[4 * a + 2], v[4 * a + 3]);
  };

  // (u, gradient row offset, table row) of position e = r*G + lane in register r: the lane
  // that loads an entry turns its bag into the offset of the bag's gradient row once, and
  // the slot's lanes take it by shuffle (rather than each of them dividing by the batch)
  int32_t ekey[kRegs];
  int64_t egoff[kRegs];
  int64_t erow[kRegs];
#pragma unroll
  for (int r = 0; r < kRegs; ++r) {
    const int e = r * G + lane;
    ekey[r] = -1;
    egoff[r] = 0;
    erow[r] = -1;
    if (e < KPS && e < len) {
      const auto en = S.entry(q0 + e);
      ekey[r] = en.key;
      uint32_t bag = (uint32_t)en.bag;
      if ((int64_t)bag >= S.num_bags) bag = 0;
      const uint32_t t = bag / (uint32_t)S.batch, b = bag - t * (uint32_t)S.batch;
      egoff[r] = (int64_t)b * S.sb + (int64_t)t * S.st;
      erow[r] = en.row;
    }
  }
  const int32_t kb = key_before<true>(S, q0);
  const int32_t ka = key_after<true>(S, q1, n);

  // all gradient rows of the slot
  int32_t kk[KPS];
  typename GV::T rv[KPS];
#pragma unroll
  for (int e = 0; e < KPS; ++e) {
    const int src_lane = lane0 + (e % G);
    kk[e] = __shfl(ekey[e / G], src_lane, 64);
    const uint64_t g = egoff[e / G];
    const int64_t goff = (int64_t)(((uint64_t)(uint32_t)__shfl((int)(uint32_t)(g >> 32), src_lane, 64) << 32) |
                                   (uint32_t)__shfl((int)(uint32_t)g, src_lane, 64));
    rv[e] = (e < len && col_ok && kk[e] != -1) ? GV::load(S, goff + c) : GV::zero();
  }

  // table rows of the segments completed inside the slot, and of the last piece
  int64_t rk[kRegs];
  TRow<MODE, CW> w[KPS];
  if constexpr (MODE != 0) {
#pragma unroll
    for (int r = 0; r < kRegs; ++r) {
      const int e = r * G + lane;
      const int32_t own = ekey[r];
      // key of position e + 1: same register one lane up, or register r + 1 of lane 0
      const int32_t up = __shfl(ekey[r], lane0 + ((lane + 1) & (G - 1)), 64);
      const int32_t wrap = (r + 1 < kRegs) ? __shfl(ekey[r + 1 < kRegs ? r + 1 : r], lane0, 64)
                                           : -1;
      const int32_t nx = (e + 1 < len) ? ((lane + 1 < G) ? up : wrap) : ka;
      const bool emit = e < KPS && e < len && own != kb && nx != own && own >= 0 &&
                        (int64_t)own < capacity;
      const bool last = e == len - 1 && own == ka && own != kb && own >= 0 &&
                        (int64_t)own < capacity;
      const int64_t key = erow[r];
      rk[r] = ((emit || last) && key >= 0 && key < sgd.total_rows) ? key : -1;
    }
#pragma unroll
    for (int e = 0; e < KPS; ++e) {
      const int64_t key = __shfl(rk[e / G], lane0 + (e % G), 64);
      w[e] = load_trow<MODE, CW>(sgd, key, c, key >= 0 && col_ok);
    }
  }

  float acc[CW];
#pragma unroll
  for (int i = 0; i < CW; ++i) acc[i] = 0.f;
#pragma unroll
  for (int e = 0; e < KPS; ++e) {
    if (e < len) {
      float x[CW];
      GV::widen(rv[e], x);
#pragma unroll
      for (int i = 0; i < CW; ++i) acc[i] += x[i];
      const int32_t k = kk[e];
      const int32_t nx = (e + 1 < len) ? kk[e + 1 < KPS ? e + 1 : e] : ka;
      if (nx != k) {                           // the piece ends at e
        if (k == kb) {                         // ... and began before the slot
          fkey = k;
          fcont = 0;
          to_lds(sm.first_row[slot], acc);
        } else if (k >= 0 && (int64_t)k < capacity) {
          if (row_grads && col_ok) {
#pragma unroll
            for (int a = 0; a < CW / 4; ++a)
              *reinterpret_cast<float4*>(row_grads + (int64_t)k * dim + c + 4 * a) =
                  make_float4(acc[4 * a], acc[4 * a + 1], acc[4 * a + 2], acc[4 * a + 3]);
          }
          if constexpr (MODE != 0) {
            const int64_t key = __shfl(rk[e / G], lane0 + (e % G), 64);
            if (key >= 0 && col_ok) store_trow<MODE, CW>(sgd, key, c, acc, w[e]);
          }
        }
#pragma unroll
        for (int i = 0; i < CW; ++i) acc[i] = 0.f;
      } else if (e == len - 1) {               // still open at the slot's end: continues
        if (k == kb) {
          fkey = k;
          fcont = 1;
          to_lds(sm.first_row[slot], acc);
        } else {
          lkey = k;
          to_lds(sm.last_row[slot], acc);
          if constexpr (MODE != 0) {
            pend.key = __shfl(rk[e / G], lane0 + (e % G), 64);
            pend.w = w[e];
          }
        }
      }
    }
  }
}

// One chunk of a reduce-by-key level.  L0: entries are sorted positions of the occurrences
// (keys from src, rows gathered from grad); otherwise entries are carries (keys may be -1 =
// empty).  The chunk's at most two carries go to out_keys / out_rows[2 * chunk + {0, 1}].
// W8 (level 0, bf16 gradient rows, VPL = 2): the lanes take 8 adjacent columns each (the
// prefetched slot with CW = 8); otherwise vector a of a lane holds columns (a G + lane) 4 ...
template <bool L0, bool W8, int G, int VPL, int MODE, int KPS, typename Src>
__device__ __forceinline__ void reduce_chunk(
    SegSmem<G, VPL>& sm, Src S, int64_t n, int64_t chunk_id, int dim, int64_t capacity,
    float* __restrict__ row_grads, const SgdTarget& sgd, int32_t* __restrict__ out_keys,
    float* __restrict__ out_rows) {
  constexpr int kSlots = kThreads / G;
  constexpr int kW = G * VPL * 4;              // floats per slot row in LDS
  const int lane = threadIdx.x & (G - 1);
  const int slot = threadIdx.x / G;
  const int64_t chunk0 = chunk_id * kSlots * KPS;
  const int64_t q0 = chunk0 + (int64_t)slot * KPS;
  const int64_t q1 = q0 + KPS < n ? q0 + KPS : n;
  const int64_t chunk1 = chunk0 + (int64_t)kSlots * KPS < n ? chunk0 + (int64_t)kSlots * KPS : n;

  static_assert(!W8 || (L0 && VPL == 2 && Src::kBf16), "8-column lanes: level 0, bf16 rows");
  constexpr bool kPrefetched = L0 && (VPL == 1 || W8);
  constexpr int CW = W8 ? 8 : 4;
  // column of vector a of this lane
  auto col = [&](int a) { return W8 ? lane * 8 + 4 * a : (a * G + lane) * 4; };
  auto write_row = [&](float* dst, const RowAcc<VPL>& r) {
#pragma unroll
    for (int a = 0; a < VPL; ++a) {
      const int c = col(a);
      if (c < dim)
        *reinterpret_cast<float4*>(dst + c) = make_float4(r.v[a][0], r.v[a][1], r.v[a][2], r.v[a][3]);
    }
  };
  auto emit_complete = [&](int32_t u, const RowAcc<VPL>& r) {
    if (u < 0 || (int64_t)u >= capacity) return;
    if (row_grads) write_row(row_grads + (int64_t)u * dim, r);
    if constexpr (MODE != 0) {
      const int64_t key = sgd.uniq ? sgd.uniq[u] : (int64_t)u;   // no uniq: keys are rows
      if (key < 0 || key >= sgd.total_rows) return;
      char* wrow = sgd.table + key * sgd.row_bytes;
#pragma unroll
      for (int a = 0; a < VPL; ++a) {
        const int c = col(a);
        if (c >= dim) continue;
        if constexpr (MODE == 1) {
          float4* wp = reinterpret_cast<float4*>(wrow + (int64_t)c * 4);
          const float4 w = *wp;
          *wp = make_float4(__builtin_fmaf(-sgd.lr, r.v[a][0], w.x),
                            __builtin_fmaf(-sgd.lr, r.v[a][1], w.y),
                            __builtin_fmaf(-sgd.lr, r.v[a][2], w.z),
                            __builtin_fmaf(-sgd.lr, r.v[a][3], w.w));
        } else {
          uint2* wp = reinterpret_cast<uint2*>(wrow + (int64_t)c * 2);
          *wp = half_updated<MODE>(sgd, key, c, r.v[a][0], r.v[a][1], r.v[a][2], r.v[a][3],
                                   *wp);
        }
      }
    }
  };

  int32_t fkey = -1, fcont = 0, lkey = -1;
  PendingRow<MODE, CW> pend;
  if constexpr (kPrefetched) {
    if (q0 < n)
      slot_prefetched<G, CW, MODE, KPS, Src>(S, q0, q1, n, dim, capacity, row_grads, sgd, sm,
                                             slot, lane, fkey, fcont, lkey, pend);
  } else if (q0 < n) {
    // Prefetch the slot's entries cooperatively: entry e is loaded by lane e % G of the slot
    // into register e / G, then broadcast with shuffles.
    constexpr int kRegs = (KPS + G - 1) / G;
    const int lane0 = (threadIdx.x & 63) & ~(G - 1);
    int32_t ekey[kRegs];
    int32_t ebag[kRegs];
#pragma unroll
    for (int r = 0; r < kRegs; ++r) {
      const int e = r * G + lane;
      const int64_t p = q0 + e;
      ekey[r] = -1;
      ebag[r] = 0;
      if (e < KPS && p < q1) {
        if constexpr (L0) {
          const auto en = S.entry(p);
          ekey[r] = en.key;
          ebag[r] = en.bag;
        } else {
          ekey[r] = S.keys[p];
        }
      }
    }
    const int32_t kb = key_before<L0>(S, q0);
    const int32_t ka = key_after<L0>(S, q1, n);
    int32_t cur = -1;
    bool cur_before = false;
    bool first_seen = false;
    RowAcc<VPL> acc;
    acc.zero();
    constexpr int kBatch = VPL == 1 ? KPS : (KPS < 8 ? KPS : 8);
#pragma unroll
    for (int b0 = 0; b0 < KPS; b0 += kBatch) {
      int32_t kk[kBatch];
      float4 rv[kBatch][VPL];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int e = b0 + u;
        const int64_t p = q0 + e;
        int64_t goff = 0;                 // L0: element offset of the bag's gradient row
        const float* rp = nullptr;        // carries: the carry row
        kk[u] = __shfl(ekey[e / G], lane0 + (e % G), 64);
        if constexpr (L0) {
          int64_t bag = __shfl(ebag[e / G], lane0 + (e % G), 64);
          if (bag < 0 || bag >= S.num_bags) bag = 0;
          const int64_t t = bag / S.batch, b = bag - t * S.batch;
          goff = b * S.sb + t * S.st;
        } else {
          rp = S.rows + p * (int64_t)S.dim;
        }
#pragma unroll
        for (int a = 0; a < VPL; ++a) {
          const int c = col(a);
          // carry rows load without waiting for their key (empty entries are skipped below)
          if (p < q1 && c < dim && (!L0 || kk[u] != -1)) {
            if constexpr (L0)
              rv[u][a] = Src::widen(S.load_raw(goff + c));
            else
              rv[u][a] = *reinterpret_cast<const float4*>(rp + c);
          } else {
            rv[u][a] = make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (kk[u] == -1) continue;
        if (kk[u] != cur) {
          if (cur != -1) {             // previous segment ended inside this slot
            if (cur_before) {
              fkey = cur;
              fcont = 0;
#pragma unroll
              for (int a = 0; a < VPL; ++a)
                *reinterpret_cast<float4*>(&sm.first_row[slot][col(a)]) =
                    make_float4(acc.v[a][0], acc.v[a][1], acc.v[a][2], acc.v[a][3]);
            } else {
              emit_complete(cur, acc);
            }
          }
          cur = kk[u];
          cur_before = !first_seen && (kk[u] == kb);
          first_seen = true;
          acc.zero();
        }
#pragma unroll
        for (int a = 0; a < VPL; ++a) {
          acc.v[a][0] += rv[u][a].x;
          acc.v[a][1] += rv[u][a].y;
          acc.v[a][2] += rv[u][a].z;
          acc.v[a][3] += rv[u][a].w;
        }
      }
    }
    if (cur != -1) {
      const bool cont = ka == cur;
      if (cur_before) {
        fkey = cur;
        fcont = cont ? 1 : 0;
#pragma unroll
        for (int a = 0; a < VPL; ++a)
          *reinterpret_cast<float4*>(&sm.first_row[slot][col(a)]) =
              make_float4(acc.v[a][0], acc.v[a][1], acc.v[a][2], acc.v[a][3]);
      } else if (cont) {
        lkey = cur;
#pragma unroll
        for (int a = 0; a < VPL; ++a)
          *reinterpret_cast<float4*>(&sm.last_row[slot][col(a)]) =
              make_float4(acc.v[a][0], acc.v[a][1], acc.v[a][2], acc.v[a][3]);
      } else {
        emit_complete(cur, acc);
      }
    }
  }
  if (lane == 0) {
    sm.first_key[slot] = fkey;
    sm.first_cont[slot] = fcont;
    sm.last_key[slot] = lkey;
  }
  if (threadIdx.x == 0) {
    sm.wg_first_key = -1;
    sm.wg_last_key = -1;
  }
  __syncthreads();

  // Join the pieces of segments that cross slot edges.  The owner of a segment is the slot
  // where it starts (its "last" piece) or, for the segment that started before this chunk,
  // slot 0.  Walking right adds the next slots' "first" pieces until one does not continue.
  const int64_t carry_base = 2 * chunk_id;
  auto walk = [&](int32_t u, int start_slot, RowAcc<VPL>& acc) -> bool {
    int j = start_slot;
    while (j < kSlots) {
      if (sm.first_key[j] != u) return true;    // defensive: cannot happen on valid input
#pragma unroll
      for (int a = 0; a < VPL; ++a) {
        const float4 x = *reinterpret_cast<const float4*>(&sm.first_row[j][col(a)]);
        acc.v[a][0] += x.x; acc.v[a][1] += x.y; acc.v[a][2] += x.z; acc.v[a][3] += x.w;
      }
      if (!sm.first_cont[j]) return true;       // ended inside slot j
      ++j;
    }
    return false;                               // runs past the end of the chunk
  };
  (void)chunk1;
  if (slot == 0 && sm.first_key[0] != -1) {
    // started before this chunk: always leaves as the chunk's first carry
    const int32_t u = sm.first_key[0];
    RowAcc<VPL> acc;
#pragma unroll
    for (int a = 0; a < VPL; ++a) {
      const float4 x = *reinterpret_cast<const float4*>(&sm.first_row[0][col(a)]);
      acc.v[a][0] = x.x; acc.v[a][1] = x.y; acc.v[a][2] = x.z; acc.v[a][3] = x.w;
    }
    if (sm.first_cont[0]) walk(u, 1, acc);
    write_row(out_rows + carry_base * dim, acc);
    if (lane == 0) sm.wg_first_key = u;
  }
  if (sm.last_key[slot] != -1) {
    const int32_t u = sm.last_key[slot];
    RowAcc<VPL> acc;
#pragma unroll
    for (int a = 0; a < VPL; ++a) {
      const float4 x = *reinterpret_cast<const float4*>(&sm.last_row[slot][col(a)]);
      acc.v[a][0] = x.x; acc.v[a][1] = x.y; acc.v[a][2] = x.z; acc.v[a][3] = x.w;
    }
    if (walk(u, slot + 1, acc)) {
      if constexpr (kPrefetched) {
        // the row was read before the join
        if (u >= 0 && (int64_t)u < capacity) {
          const int c = col(0);
          float g[CW];
#pragma unroll
          for (int a = 0; a < VPL; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) g[4 * a + i] = acc.v[a][i];
          if (row_grads && c < dim) write_row(row_grads + (int64_t)u * dim, acc);
          if constexpr (MODE != 0)
            if (pend.key >= 0 && c < dim) store_trow<MODE, CW>(sgd, pend.key, c, g, pend.w);
        }
      } else {
        emit_complete(u, acc);
      }
    } else {
      write_row(out_rows + (carry_base + 1) * dim, acc);
      if (lane == 0) sm.wg_last_key = u;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && out_keys) {
    out_keys[carry_base] = sm.wg_first_key;
    out_keys[carry_base + 1] = sm.wg_last_key;
  }
  (void)kW;
}

// One reduce-by-key level, a chunk per block.  With `ticket`, the level is the last but one:
// its carries fit one chunk, and the block that finishes last reduces them as the final
// level (its writes published by a device-scope fence before the ticket; the finisher
// fences again before it reads them), which saves a launch.  The L0 kernel, which always
// precedes, zeroes the ticket.
template <bool L0, bool W8, int G, int VPL, int MODE, int KPS, typename Src>
__global__ __launch_bounds__(kThreads) void segreduce_kernel(
    Src S, int64_t n, int dim, int64_t capacity, float* __restrict__ row_grads, SgdTarget sgd,
    int32_t* __restrict__ out_keys, float* __restrict__ out_rows, uint32_t* __restrict__ ticket,
    float* __restrict__ spare_rows) {
  __shared__ SegSmem<G, VPL> sm;
  __shared__ uint32_t finisher;
  if constexpr (L0) {
    if (ticket && blockIdx.x == 0 && threadIdx.x == 0) *ticket = 0u;
  }
  reduce_chunk<L0, W8, G, VPL, MODE, KPS, Src>(sm, S, n, (int64_t)blockIdx.x, dim, capacity,
                                               row_grads, sgd, out_keys, out_rows);
  if constexpr (!L0) {
    if (ticket) {
      __syncthreads();
      if (threadIdx.x == 0) {
        __threadfence();
        finisher = atomicAdd(ticket, 1u) == gridDim.x - 1 ? 1u : 0u;
      }
      __syncthreads();
      if (finisher) {
        __threadfence();
        const LnSource fin{out_keys, out_rows, dim};
        reduce_chunk<false, false, G, VPL, MODE, KPS, LnSource>(sm, fin, 2 * (int64_t)gridDim.x, 0, dim,
                                                    capacity, row_grads, sgd, nullptr,
                                                    spare_rows);
      }
    }
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdWs {
  int32_t* bag_of;
  int4* src;
  uint32_t* ticket;        // finish-level ticket (zeroed by the L0 kernel)
  int32_t* ckeys[2];
  float* crows[2];
  size_t bytes;
};

// Lanes per row of level 0 when bf16 gradient rows are read 8 columns (16 bytes) per lane:
// the power of two covering dim / 8 (at most 64), or 0 where that does not apply (fp32
// gradient rows, dim not a multiple of 8, or rows of more than 512 values).
int level0_w8_lanes(bool bf16_grads, int dim) {
  if (!bf16_grads || dim % 8 != 0 || dim / 8 > 64) return 0;
  int G = 1;
  while (G < dim / 8) G <<= 1;
  return G;
}

int64_t chunk_positions(int dim, int kps) {
  const RowGeom rg = row_geom(dim / 4);
  return (int64_t)(kThreads / rg.G) * kps;
}

BwdWs carve(void* base, int64_t n, int dim) {
  BwdWs w{};
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t sz) {
    char* p = b ? b + off : nullptr;
    off += align256(sz);
    return p;
  };
  const int64_t chunk = chunk_positions(dim, kMinSlotDepth);
  const int64_t c1 = 2 * ((n + chunk - 1) / chunk);   // carries out of level 0 (largest)
  w.bag_of = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)n));
  w.src = reinterpret_cast<int4*>(take(sizeof(int4) * (size_t)n));
  w.ticket = reinterpret_cast<uint32_t*>(take(256));
  for (int k = 0; k < 2; ++k) {
    w.ckeys[k] = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)(c1 + 2)));
    w.crows[k] = reinterpret_cast<float*>(take(sizeof(float) * (size_t)(c1 + 2) * dim));
  }
  w.bytes = off;
  return w;
}

// The carries and the ticket alone (the grouping comes from the unique's sorted_src).
BwdWs carve_carries(void* base, int64_t n, int dim) {
  BwdWs w{};
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t sz) {
    char* p = b ? b + off : nullptr;
    off += align256(sz);
    return p;
  };
  const int64_t chunk = chunk_positions(dim, kMinSlotDepth);
  const int64_t c1 = 2 * ((n + chunk - 1) / chunk);
  w.ticket = reinterpret_cast<uint32_t*>(take(256));
  for (int k = 0; k < 2; ++k) {
    w.ckeys[k] = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (size_t)(c1 + 2)));
    w.crows[k] = reinterpret_cast<float*>(take(sizeof(float) * (size_t)(c1 + 2) * dim));
  }
  w.bytes = off;
  return w;
}

}  // namespace

// Scratch of the backward that allocates nothing (launch_embbag_bwd_noalloc): the carries
// of the reduce-by-key levels and the finisher's ticket, for callers that cannot allocate.
// Each GPU the library runs on holds its own copy until the process ends; every call on a
// GPU shares it, so calls that overlap on one GPU race.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this GPU's scratch, taken once per device with that device current.
// (The name `scratch` in host code is a host-side stand-in, never a device address.)
hipError_t scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

size_t embbag_bwd_workspace_bytes(int64_t nnz, int dim) { return carve(nullptr, nnz, dim).bytes; }
size_t embbag_bwd_noalloc_bytes(int64_t nnz, int dim) {
  return carve_carries(nullptr, nnz, dim).bytes;
}


#define CTR_SEG_DISPATCH(G_, VPL_, ...)                                     \
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

// capacity: keys are below it (the distinct rows' count bound nnz, or the table's rows when
// the keys are rows).
template <int MODE, typename L0S>
static hipError_t segreduce_levels(const L0S& s0, int64_t nnz, int64_t capacity, int dim,
                                   float* row_grads, const SgdTarget& sgd, BwdWs& w,
                                   hipStream_t s, void* l0_begin, void* l0_end) {
  hipError_t e = record_mark(l0_begin, s);
  if (e != hipSuccess) return e;
  const RowGeom rg = row_geom(dim / 4);
  constexpr int KPS = slot_depth<L0S::kBf16>();
  const int64_t chunk = chunk_positions(dim, KPS);
  // level 0: bf16 gradient rows in 8-column lanes where the row allows (level0_lanes)
  const int g8 = level0_w8_lanes(L0S::kBf16, dim);
  const int64_t chunk0 = g8 ? (int64_t)(kThreads / g8) * KPS : chunk;
  int64_t blocks = (nnz + chunk0 - 1) / chunk0;
  int cur = 0;
  if constexpr (L0S::kBf16) {
    if (g8) {
      CTR_SEG_DISPATCH(g8, 1, {
        (void)VPL;
        segreduce_kernel<true, true, G, 2, MODE, KPS, L0S><<<(unsigned)blocks, kThreads, 0, s>>>(
            s0, nnz, dim, capacity, row_grads, sgd, blocks > 1 ? w.ckeys[cur] : nullptr,
            w.crows[cur], w.ticket, nullptr);
      });
    }
  }
  if (!g8) {
    CTR_SEG_DISPATCH(rg.G, rg.VPL, {
      segreduce_kernel<true, false, G, VPL, MODE, KPS, L0S><<<(unsigned)blocks, kThreads, 0, s>>>(
          s0, nnz, dim, capacity, row_grads, sgd, blocks > 1 ? w.ckeys[cur] : nullptr,
          w.crows[cur], w.ticket, nullptr);
    });
  }
  e = record_mark(l0_end, s);
  CTR_SEG_DISPATCH(rg.G, rg.VPL, {
    int64_t len = nnz;
    while (e == hipSuccess && blocks > 1) {
      len = 2 * blocks;
      blocks = (len + chunk - 1) / chunk;
      LnSource sn{w.ckeys[cur], w.crows[cur], dim};
      // a level whose carries fit one chunk finishes the tree itself
      const bool fold = blocks > 1 && 2 * blocks <= chunk && blocks <= kFoldBlocks;
      segreduce_kernel<false, false, G, VPL, MODE, KPS, LnSource><<<(unsigned)blocks, kThreads, 0, s>>>(
          sn, len, dim, capacity, row_grads, sgd, blocks > 1 ? w.ckeys[cur ^ 1] : nullptr,
          w.crows[cur ^ 1], fold ? w.ticket : nullptr, w.crows[cur]);
      cur ^= 1;
      if (fold) break;
    }
  });
  return e;
}

namespace {
// The gradient source of level 0 and the reduce-by-key levels, into the carved workspace w.
hipError_t embbag_bwd_levels(const BwdWs& w, const void* grad, bool grad_bf16, int64_t sb,
                             int64_t st, const int64_t* offsets, int64_t batch,
                             int32_t num_tables, int dim, int64_t nnz, const int32_t* perm,
                             const int32_t* inverse, const void* sorted_src, bool src_rows,
                             float* row_grads, void* table, int sgd_mode, int64_t total_rows,
                             const int64_t* uniq, float lr, uint64_t seed, hipStream_t s,
                             void* l0_begin, void* l0_end) {
  BwdWs wm = w;
  const int64_t num_bags = (int64_t)num_tables * batch;

  const void* src = sorted_src;
  if (!src) {
    // (u, bag) per sorted position from perm and inverse: expand the bags, then gather.
    const int64_t waves = (num_bags + 63) / 64;
    const int64_t blocks = (waves + 3) / 4;
    bag_of_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(offsets, num_bags, nnz, w.bag_of);
    seg_src_kernel<<<(unsigned)((nnz + kThreads - 1) / kThreads), kThreads, 0, s>>>(
        perm, inverse, w.bag_of, nnz, w.src);
    src = w.src;
  }

  // row entries: the keys are the table rows (below total_rows) and need no uniq
  SgdTarget sgd{static_cast<char*>(table), total_rows,
                (int64_t)dim * (sgd_mode >= 2 ? 2 : 4), src_rows ? nullptr : uniq, lr, seed};
  const int64_t cap = src_rows ? total_rows : nnz;
  auto levels = [&](const auto& s0) -> hipError_t {
    using S0 = std::decay_t<decltype(s0)>;
    switch (sgd_mode) {
      case 1: return segreduce_levels<1, S0>(s0, nnz, cap, dim, row_grads, sgd, wm, s, l0_begin, l0_end);
      case 2: return segreduce_levels<2, S0>(s0, nnz, cap, dim, row_grads, sgd, wm, s, l0_begin, l0_end);
      case 3: return segreduce_levels<3, S0>(s0, nnz, cap, dim, row_grads, sgd, wm, s, l0_begin, l0_end);
      case 4: return segreduce_levels<4, S0>(s0, nnz, cap, dim, row_grads, sgd, wm, s, l0_begin, l0_end);
      case 5: return segreduce_levels<5, S0>(s0, nnz, cap, dim, row_grads, sgd, wm, s, l0_begin, l0_end);
      default:
        // row gradients are indexed by u, which row entries do not carry (the caller checks)
        if constexpr (S0::kRows) return hipErrorInvalidValue;
        else return segreduce_levels<0, S0>(s0, nnz, cap, dim, row_grads, sgd, wm, s, l0_begin, l0_end);
    }
  };
  hipError_t e;
  if (src_rows)
    e = grad_bf16 ? levels(L0SourceT<true, true>{src, grad, sb, st, batch, num_bags})
                  : levels(L0SourceT<false, true>{src, grad, sb, st, batch, num_bags});
  else
    e = grad_bf16 ? levels(L0SourceB{src, grad, sb, st, batch, num_bags})
                  : levels(L0Source{src, grad, sb, st, batch, num_bags});
  if (e != hipSuccess) return e;
  return hipGetLastError();
}
}  // namespace

hipError_t launch_embbag_bwd(const void* grad, bool grad_bf16, int64_t sb, int64_t st,
                             const int64_t* offsets,
                             int64_t batch, int32_t num_tables, int dim, int64_t nnz,
                             const int32_t* perm, const int32_t* inverse, const void* sorted_src,
                             bool src_rows, const int32_t* num_unique, float* row_grads,
                             void* table,
                             int sgd_mode, int64_t total_rows, const int64_t* uniq, float lr,
                             uint64_t seed, void* workspace, hipStream_t s, void* l0_begin,
                             void* l0_end) {
  (void)num_unique;
  if (nnz == 0) {                          // nothing to reduce; the marks still bracket it
    const hipError_t e = record_mark(l0_begin, s);
    return e == hipSuccess ? record_mark(l0_end, s) : e;
  }
  BwdWs w = carve(workspace, nnz, dim);
  return embbag_bwd_levels(w, grad, grad_bf16, sb, st, offsets, batch, num_tables, dim, nnz, perm,
                           inverse, sorted_src, src_rows, row_grads, table, sgd_mode, total_rows,
                           uniq, lr, seed, s, l0_begin, l0_end);
}

hipError_t launch_embbag_bwd_noalloc(const void* grad, bool grad_bf16, int64_t sb, int64_t st,
                                     const int64_t* offsets, int64_t batch, int32_t num_tables,
                                     int dim, int64_t nnz, const void* sorted_src,
                                     bool src_rows, float* row_grads, void* table, int sgd_mode,
                                     int64_t total_rows, const int64_t* uniq, float lr,
                                     uint64_t seed, hipStream_t s) {
  if (nnz == 0) return hipSuccess;
  void* base = nullptr;
  const hipError_t e = scratch_on_current_device(&base);
  if (e != hipSuccess) return e;
  BwdWs w = carve_carries(base, nnz, dim);   // fits: the caller checked the size
  return embbag_bwd_levels(w, grad, grad_bf16, sb, st, offsets, batch, num_tables, dim, nnz,
                           nullptr, nullptr, sorted_src, src_rows, row_grads, table, sgd_mode,
                           total_rows, uniq, lr, seed, s, nullptr, nullptr);
}

}  // namespace ctr
