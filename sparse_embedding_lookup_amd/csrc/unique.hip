// unique.hip -- batch ID deduplication on gfx950: key formation, a stable LSD radix sort
// over only the live key bits, and the unique / inverse / segment finalize.
//
// Method: "How TensorNet Supercharges Sparse Feature Training on TensorFlow", section
// "Core Optimizations": collect the batch's IDs, sort them and give each distinct ID a
// contiguous index.  The sort is ours: reduce-then-scan LSD radix, digits of up to 8 bits
// spread evenly over the passes (a 28-bit row key takes four 7-bit passes: with 2048-key
// tiles, wider digits leave too few keys per digit for the output runs to coalesce), the
// wider ones last (22 bits: 7, 7, 8), where the earlier passes have already gathered a
// power-law batch's repeated rows into runs that write out whole:
//   keys      one wave per 64 bags forms the keys of their occurrences (the bag of each
//             occurrence comes from a shuffle binary search over the 64 bag ends, so the
//             table and the bag are known without a search over all offsets)
//   upsweep   each block counts digits of its contiguous range (wave-aggregated counts)
//   scan      one block per digit scans that digit's per-block counts (with few blocks the
//             downsweep sums the digit's row of counts itself, with 16-byte loads)
//   downsweep each block ranks its tiles stably with wave64 ballot "multisplit" (one
//             ballot per digit bit gives the mask of lanes holding the same digit), stages
//             the tile in LDS in digit order and writes it out in runs per digit.
// Tables as segments: when the caller gives the largest table's row count, the occurrences
// of one table are contiguous (bags are table-major), and table t's keys are row_base[t]
// plus a local row below 2^L, the sort key is (t << L) | local and every radix pass sorts
// the L local bits within each table's range only (a pass's blocks each hold one table's
// stretch; a block's digit offsets are its table's start plus the prefixes within that
// table).  The table bits are never sorted: Large's 28-bit keys take three passes of local
// rows instead of four, and the finalize rebuilds row_base[t] + local.
// The payload is the occurrence index alone.  When bags are given, key formation also writes
// each occurrence's bag in occurrence order, and the finalize reads it through the sorted
// occurrence index to emit (distinct-row index, bag) per sorted position for the backward's
// reduce-by-key: the sorted positions of one table read one table's stretch of that array, a
// few MB that the caches hold, instead of a third array moved through every pass.  No
// inter-block waiting anywhere.
#include <utility>

#include "ctr_internal.h"

namespace ctr {
namespace {

constexpr int kThreads = 256;                 // 4 waves
constexpr int kMaxBits = 8;                   // widest digit (wider digits scatter worse)
constexpr int kBuckets = 1 << kMaxBits;
constexpr int kMaxBlocks = 1024;              // radix blocks (ranges) per pass
constexpr int kFinTile = 2048;                // positions per finalize block
constexpr int kFusedScanBlocks = 64;          // up to this many blocks, no scan kernel

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

// Mask of the lanes in `active` whose digit equals this lane's digit.
__device__ __forceinline__ uint64_t match_digit(uint32_t d, int nbits, uint64_t active) {
  uint64_t m = active;
  for (int b = 0; b < nbits; ++b) {
    const uint32_t bit = (d >> b) & 1u;
    const uint64_t bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

// Radix block of the table-segmented sort: the table it belongs to (-1: no work), the
// table's first block and the next table's first block, the table's first position, and the
// block's range of positions.
constexpr int kMaxSegTables = 512;
struct SegBlock {
  int32_t seg, first, next, pad;
  int64_t seg_beg, beg, end;
};

// One block: each table's stretch of positions [offsets[t*batch], offsets[(t+1)*batch]) is
// cut into ceil(len / per_block) blocks; block b learns its table, its range and the first
// blocks of its table and the next.
__global__ __launch_bounds__(1024) void seg_blocks_kernel(const int64_t* __restrict__ offsets,
                                                          int64_t batch, int num_tables,
                                                          int64_t n, int64_t per_block,
                                                          int nblocks,
                                                          SegBlock* __restrict__ blk) {
  __shared__ int64_t start[kMaxSegTables + 1];
  __shared__ int32_t first[kMaxSegTables + 1];
  for (int t = threadIdx.x; t <= num_tables; t += blockDim.x)
    start[t] = clamp64(offsets[(int64_t)t * batch], 0, n);
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t acc = 0;
    for (int t = 0; t < num_tables; ++t) {
      first[t] = acc;
      const int64_t len = start[t + 1] > start[t] ? start[t + 1] - start[t] : 0;
      acc += (int32_t)((len + per_block - 1) / per_block);
    }
    first[num_tables] = acc;
  }
  __syncthreads();
  for (int b = threadIdx.x; b < nblocks; b += blockDim.x) {
    SegBlock m{-1, 0, 0, 0, 0, 0, 0};
    if (b < first[num_tables]) {
      int lo = 0, hi = num_tables - 1;          // last table whose first block is <= b
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (first[mid] <= b) lo = mid; else hi = mid - 1;
      }
      const int64_t beg = start[lo] + (int64_t)(b - first[lo]) * per_block;
      const int64_t end = beg + per_block < start[lo + 1] ? beg + per_block : start[lo + 1];
      m = SegBlock{lo, first[lo], first[lo + 1], 0, start[lo], beg, end};
    }
    blk[b] = m;
  }
}

// Exclusive scan of one uint32 per thread over a 256-thread block; returns the exclusive
// prefix and stores the block total in *total.  `tmp` holds 4 words of LDS.
__device__ __forceinline__ uint32_t block_excl_scan_256(uint32_t v, uint32_t* tmp,
                                                        uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t t = tmp[w];
    if (w < wave) base += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__device__ __forceinline__ int64_t floor_mod(int64_t id, int64_t m) {
  if (m > 0) {
    id %= m;
    if (id < 0) id += m;
  }
  return id;
}

// --------------------------------------------------------------------------- a1: keys
// Bags known: `parts` waves share one group of 64 consecutive bags; lane l holds the end of
// bag s0 + l and every occurrence finds its bag by a 6-step binary search over those ends
// (shuffles); each wave takes every parts-th stretch of 64 occurrences of the group.
// B16: the bag is stored as its sample index (bag - table * batch, batch <= 65536) in 16 bits,
// which halves the array the finalize reads through the occurrence index; the table comes
// back from the key.
template <bool ID64, typename K, bool B16>
__global__ __launch_bounds__(kThreads) void form_keys_bags_kernel(
    const void* __restrict__ ids, int64_t n, const int64_t* __restrict__ offsets, int64_t batch,
    int64_t num_bags, const int64_t* __restrict__ row_base, int64_t modulus, uint64_t flip,
    int parts, int seg_bits, K* __restrict__ keys, void* __restrict__ bags) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t s0 = (wave / parts) * 64;
  const int part = (int)(wave % parts);
  if (s0 >= num_bags) return;
  const int64_t s = s0 + lane;
  const int64_t my_end = s < num_bags ? clamp64(offsets[s + 1], 0, n) : INT64_MAX;
  const int64_t beg = clamp64(offsets[s0], 0, n);
  const int64_t last = s0 + 64 < num_bags ? s0 + 64 : num_bags;
  const int64_t end = clamp64(offsets[last], beg, n);
  for (int64_t i0 = beg + (int64_t)part * 64; i0 < end; i0 += (int64_t)parts * 64) {
    const int64_t i = i0 + lane;
    int l = 0;
#pragma unroll
    for (int step = 32; step > 0; step >>= 1) {
      const int64_t e = __shfl(my_end, l + step - 1, 64);
      if (e <= i) l += step;
    }
    if (i < end) {
      const int64_t bag = s0 + l;
      const int64_t id = ID64 ? static_cast<const int64_t*>(ids)[i]
                              : (int64_t) static_cast<const int32_t*>(ids)[i];
      int64_t key = floor_mod(id, modulus);
      if (seg_bits) key = (int64_t)(((uint64_t)(bag / batch) << seg_bits) | (uint64_t)key);
      else if (row_base) key += row_base[bag / batch];
      keys[i] = (K)((uint64_t)key ^ flip);
      if constexpr (B16)
        static_cast<uint16_t*>(bags)[i] = (uint16_t)(bag - (bag / batch) * batch);
      else
        static_cast<uint32_t*>(bags)[i] = (uint32_t)bag;
    }
  }
}

// No bags: each occurrence is its own bag.
template <bool ID64, typename K>
__global__ __launch_bounds__(kThreads) void form_keys_flat_kernel(const void* __restrict__ ids,
                                                                  int64_t n, int64_t modulus,
                                                                  uint64_t flip,
                                                                  K* __restrict__ keys) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    const int64_t id = ID64 ? static_cast<const int64_t*>(ids)[i]
                            : (int64_t) static_cast<const int32_t*>(ids)[i];
    keys[i] = (K)((uint64_t)floor_mod(id, modulus) ^ flip);
  }
}

// --------------------------------------------------------------------------- upsweep
// Digit counts of each block's contiguous range; hist is digit-major: hist[digit * ld + block]
// (ld = block count rounded up to 4), so one digit's counts over the blocks are contiguous.
constexpr int kUpU = 4;   // keys in flight per thread in the upsweep

// Range of radix block b: the segment map's (table-segmented sort), else b * per_block.
__device__ __forceinline__ void block_range(const SegBlock* blk, int64_t per_block, int64_t n,
                                            int64_t* beg, int64_t* end) {
  if (blk) {
    const SegBlock& m = blk[blockIdx.x];
    *beg = m.seg < 0 ? 0 : m.beg;
    *end = m.seg < 0 ? 0 : m.end;
  } else {
    *beg = (int64_t)blockIdx.x * per_block;
    *end = *beg + per_block < n ? *beg + per_block : n;
  }
}

// One count per live lane into the wave's bins.  The LDS serves the lanes of one atomic that
// hit one address one after another, and once a pass has grouped equal keys, a power-law
// batch's hot row fills most of a wave with one digit: the lanes holding the first live
// lane's digit are counted by that lane alone, with one add of their number, and only the
// other lanes add their own one.  Called by every lane of the wave.
__device__ __forceinline__ void count_digit(uint32_t* bins, uint32_t d, bool live) {
  const uint64_t act = __ballot(live);
  if (act == 0ull) return;
  const int leader = __builtin_ctzll(act);
  const uint32_t f = (uint32_t)__builtin_amdgcn_readlane((int)d, leader);
  const bool same = live && d == f;
  const uint64_t grp = __ballot(same);
  if ((threadIdx.x & 63) == leader) atomicAdd(&bins[f], (uint32_t)__popcll(grp));
  else if (live && !same) atomicAdd(&bins[d], 1u);
}

template <typename K>
__global__ __launch_bounds__(kThreads) void radix_upsweep_kernel(
    const K* __restrict__ keys, int64_t n, int shift, int nbits, int64_t per_block,
    const SegBlock* __restrict__ blk, uint32_t* __restrict__ hist, int ld) {
  __shared__ uint32_t cnt[4][kBuckets];
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * kBuckets; i += kThreads) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const uint32_t mask = (1u << nbits) - 1u;
  int64_t beg, end;
  block_range(blk, per_block, n, &beg, &end);
  // Counting needs no order: LDS atomic adds into the wave's own bins (waves never
  // contend; count_digit takes the largest group of lanes sharing a digit out of the
  // serialised adds).  Keys are read as 16-byte vectors, kUpU per thread issued before any
  // is counted; the keys before the first 16-byte boundary of the range and after its last
  // one are read one at a time.
  constexpr int V = 16 / (int)sizeof(K);
  const int64_t vbeg = ((beg + V - 1) / V) * V < end ? ((beg + V - 1) / V) * V : end;
  const int64_t vend = vbeg + ((end - vbeg) / V) * V;
  for (int64_t e = beg + threadIdx.x; e < vbeg; e += kThreads)
    atomicAdd(&cnt[wave][(uint32_t)(keys[e] >> shift) & mask], 1u);
  for (int64_t base = vbeg; base < vend; base += (int64_t)kThreads * kUpU * V) {
    uint4 raw[kUpU];
#pragma unroll
    for (int j = 0; j < kUpU; ++j) {
      const int64_t e = base + ((int64_t)j * kThreads + threadIdx.x) * V;
      raw[j] = *reinterpret_cast<const uint4*>(keys + (e < vend ? e : vend - V));
    }
#pragma unroll
    for (int j = 0; j < kUpU; ++j) {
      const bool live = base + ((int64_t)j * kThreads + threadIdx.x) * V < vend;
      const K* kv = reinterpret_cast<const K*>(&raw[j]);
#pragma unroll
      for (int v = 0; v < V; ++v) count_digit(cnt[wave], (uint32_t)(kv[v] >> shift) & mask, live);
    }
  }
  for (int64_t e = vend + threadIdx.x; e < end; e += kThreads)
    atomicAdd(&cnt[wave][(uint32_t)(keys[e] >> shift) & mask], 1u);
  __syncthreads();
  const int d = threadIdx.x;
  hist[(int64_t)d * ld + blockIdx.x] = cnt[0][d] + cnt[1][d] + cnt[2][d] + cnt[3][d];
}

// --------------------------------------------------------------------------- scan
// Many blocks: block d scans digit d's counts over the blocks (exclusive, in place) and
// stores the digit total.  (With few blocks the downsweep does this itself.)
__global__ __launch_bounds__(kThreads) void radix_scan_kernel(uint32_t* __restrict__ hist,
                                                              int nblocks, int ld,
                                                              uint32_t* __restrict__ totals) {
  __shared__ uint32_t tmp[4];
  const int d = blockIdx.x;
  const int per = (nblocks + kThreads - 1) / kThreads;   // <= 4
  const int b0 = threadIdx.x * per;
  uint32_t local[4] = {0, 0, 0, 0};
  uint32_t sum = 0;
  for (int j = 0; j < per; ++j) {
    const int k = b0 + j;
    local[j] = k < nblocks ? hist[(int64_t)d * ld + k] : 0u;
    sum += local[j];
  }
  uint32_t total;
  uint32_t run = block_excl_scan_256(sum, tmp, &total);
  for (int j = 0; j < per; ++j) {
    const int k = b0 + j;
    if (k < nblocks) hist[(int64_t)d * ld + k] = run;
    run += local[j];
  }
  if (threadIdx.x == 0) totals[d] = total;
}

// --------------------------------------------------------------------------- downsweep
template <typename K, int ITEMS, bool B16>
struct DownsweepSmem {
  K keys[kThreads * ITEMS];
  uint32_t vals[kThreads * ITEMS];
  uint16_t bags[B16 ? kThreads * ITEMS : 2];
  uint32_t wcnt[4][kBuckets];
  uint32_t run[kBuckets];
  uint32_t tstart[kBuckets];
  uint32_t tcount[kBuckets];
  uint32_t tmp[4];
};

// IDENT: payload of pass 0 is the element index.  VAL: the occurrence payload is carried at
// all (not when the caller wants neither the inverse map nor the permutation and the bags
// ride along: then keys and bags alone move).  FUSED: few blocks, so this block sums the
// digit counts of the blocks before it itself instead of reading a separate scan's output.
// B16: a second payload, the occurrence's 16-bit sample index, rides along (pass 0 reads it
// in occurrence order, which is the element order then).
// blk (table-segmented sort): the block's table, range and first blocks; its digit
// offsets are the table's first position plus prefixes within the table, read off the
// global per-digit scan as differences from the table's first block.
template <typename K, int ITEMS, bool IDENT, bool FUSED, bool B16, bool VAL>
__global__ __launch_bounds__(kThreads) void radix_downsweep_kernel(
    const K* __restrict__ keys_in, const uint32_t* __restrict__ vals_in,
    const uint16_t* __restrict__ bags_in, K* __restrict__ keys_out,
    uint32_t* __restrict__ vals_out, uint16_t* __restrict__ bags_out, int64_t n, int shift,
    int nbits, int64_t per_block, const SegBlock* __restrict__ blk,
    const uint32_t* __restrict__ hist, const uint32_t* __restrict__ totals, int nblocks,
    int ld) {
  constexpr int kT = kThreads * ITEMS;
  __shared__ DownsweepSmem<K, ITEMS, B16> sm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t mask = (1u << nbits) - 1u;

  // Global start of each digit for this block: all digits before it, then the same digit in
  // the blocks before it.
  {
    const int d = threadIdx.x;
    uint32_t tot, before;
    if (FUSED) {
      // digit d's counts over all blocks are one contiguous row: 16-byte loads, all issued
      // before any is summed
      tot = 0;
      before = 0;
      const uint4* row = reinterpret_cast<const uint4*>(hist + (int64_t)d * ld);
      const int me = (int)blockIdx.x;
#pragma unroll 8
      for (int g4 = 0; g4 < ld / 4; ++g4) {
        const uint4 v = row[g4];
        const uint32_t c[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int g = 4 * g4 + j;
          const uint32_t x = g < nblocks ? c[j] : 0u;
          tot += x;
          before += g < me ? x : 0u;
        }
      }
    } else if (blk) {
      const SegBlock& m = blk[blockIdx.x];
      const int64_t row = (int64_t)d * ld;
      const uint32_t h0 = m.seg < 0 ? 0u : hist[row + m.first];
      before = m.seg < 0 ? 0u : hist[row + blockIdx.x] - h0;
      tot = m.seg < 0 ? 0u : (m.next < nblocks ? hist[row + m.next] : totals[d]) - h0;
    } else {
      tot = totals[d];
      before = hist[(int64_t)d * ld + blockIdx.x];
    }
    uint32_t all;
    const uint32_t base = blk ? (uint32_t)blk[blockIdx.x].seg_beg : 0u;
    sm.run[d] = base + block_excl_scan_256(tot, sm.tmp, &all) + before;
  }
  __syncthreads();

  int64_t beg, end;
  block_range(blk, per_block, n, &beg, &end);
  const uint64_t lt = lanemask_lt();

  for (int64_t tile = beg; tile < end; tile += kT) {
    K key[ITEMS];
    uint32_t val[ITEMS];
    uint16_t bag[ITEMS];
    uint32_t rank[ITEMS];
    bool valid[ITEMS];
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int64_t e = tile + (int64_t)wave * 64 * ITEMS + k * 64 + lane;
      valid[k] = e < end;
      key[k] = valid[k] ? keys_in[e] : (K)0;
      val[k] = (VAL && valid[k]) ? (IDENT ? (uint32_t)e : vals_in[e]) : 0u;
      bag[k] = (B16 && valid[k]) ? bags_in[e] : (uint16_t)0;
    }
    for (int d = lane; d < kBuckets; d += 64) sm.wcnt[wave][d] = 0;
    __builtin_amdgcn_wave_barrier();
    // Rank within the wave: the lanes of an item that share a digit (ballot multisplit) add
    // their count to the wave's bin with one returning LDS atomic from their lowest lane.  A
    // wave's LDS operations complete in issue order, so item k's atomics see items 0..k-1,
    // and every item's atomic is in flight before any result is used.
    uint64_t mm[ITEMS];
    uint32_t pre[ITEMS];
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const uint32_t d = (uint32_t)(key[k] >> shift) & mask;
      const uint64_t active = __ballot(valid[k]);
      mm[k] = match_digit(d, nbits, active);
      pre[k] = 0u;
      if (valid[k] && (mm[k] & lt) == 0ull)
        pre[k] = atomicAdd(&sm.wcnt[wave][d], (uint32_t)__popcll(mm[k]));
    }
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int leader = mm[k] ? (int)__builtin_ctzll(mm[k]) : 0;   // lowest lane of the digit
      rank[k] = (uint32_t)__shfl((int)pre[k], leader, 64) + (uint32_t)__popcll(mm[k] & lt);
    }
    __syncthreads();
    {
      const int d = threadIdx.x;
      const uint32_t c0 = sm.wcnt[0][d], c1 = sm.wcnt[1][d], c2 = sm.wcnt[2][d],
                     c3 = sm.wcnt[3][d];
      sm.wcnt[0][d] = 0;
      sm.wcnt[1][d] = c0;
      sm.wcnt[2][d] = c0 + c1;
      sm.wcnt[3][d] = c0 + c1 + c2;
      const uint32_t cnt = c0 + c1 + c2 + c3;
      sm.tcount[d] = cnt;
      uint32_t all;
      sm.tstart[d] = block_excl_scan_256(cnt, sm.tmp, &all);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      if (valid[k]) {
        const uint32_t d = (uint32_t)(key[k] >> shift) & mask;
        const uint32_t pos = sm.tstart[d] + sm.wcnt[wave][d] + rank[k];
        sm.keys[pos] = key[k];
        if constexpr (VAL) sm.vals[pos] = val[k];
        if constexpr (B16) sm.bags[pos] = bag[k];
      }
    }
    __syncthreads();
    const int tile_n = (int)((end - tile) < kT ? (end - tile) : kT);
    for (int q = threadIdx.x; q < tile_n; q += kThreads) {
      const K kk = sm.keys[q];
      const uint32_t d = (uint32_t)(kk >> shift) & mask;
      const uint32_t o = sm.run[d] + (uint32_t)q - sm.tstart[d];
      keys_out[o] = kk;
      if constexpr (VAL) vals_out[o] = sm.vals[q];
      if constexpr (B16) bags_out[o] = sm.bags[q];
    }
    __syncthreads();
    sm.run[threadIdx.x] += sm.tcount[threadIdx.x];
    __syncthreads();
  }
}

// --------------------------------------------------------------------------- finalize
// Positions are striped: in round j a 256-thread block covers 256 consecutive positions, so
// every load and store is coalesced; a head is a position whose key differs from the one
// before, and ranks come from wave ballots (popcount of the heads before a lane).
constexpr int kFinRounds = kFinTile / kThreads;     // 8
constexpr int kFusedHeadTiles = 1024;               // up to this many tiles, no scan kernel

template <typename K>
__device__ __forceinline__ bool is_head(const K* __restrict__ sk, int64_t p, int64_t n, K* key) {
  if (p >= n) return false;
  *key = sk[p];
  return p == 0 || *key != sk[p - 1];
}

template <typename K>
__global__ __launch_bounds__(kThreads) void heads_count_kernel(const K* __restrict__ sk,
                                                               int64_t n,
                                                               uint32_t* __restrict__ tile_heads) {
  __shared__ uint32_t wsum[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kFinTile;
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < kFinRounds; ++j) {
    K k;
    const bool h = is_head(sk, t0 + (int64_t)j * kThreads + threadIdx.x, n, &k);
    c += (uint32_t)__popcll(__ballot(h));
  }
  if (lane == 0) wsum[wave] = c;
  __syncthreads();
  if (threadIdx.x == 0) tile_heads[blockIdx.x] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

// One block of 1024 threads: exclusive scan of the per-tile head counts; publishes U.
__global__ __launch_bounds__(1024) void heads_scan_kernel(uint32_t* __restrict__ tile_heads,
                                                          int64_t ntiles, int64_t n,
                                                          int32_t* __restrict__ num_unique,
                                                          int32_t* __restrict__ seg_offsets) {
  __shared__ uint32_t wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t per = (ntiles + 1023) / 1024;
  const int64_t b0 = (int64_t)threadIdx.x * per;
  uint32_t s = 0;
  for (int64_t j = 0; j < per; ++j)
    if (b0 + j < ntiles) s += tile_heads[b0 + j];
  uint32_t x = s;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) base += wsum[w];
    tot += wsum[w];
  }
  uint32_t run = base + x - s;
  for (int64_t j = 0; j < per; ++j)
    if (b0 + j < ntiles) {
      const uint32_t v = tile_heads[b0 + j];
      tile_heads[b0 + j] = run;
      run += v;
    }
  if (threadIdx.x == 0) {
    *num_unique = (int32_t)tot;
    if (seg_offsets) seg_offsets[tot] = (int32_t)n;
  }
}

// sorted_src[p] = (distinct-row index of position p, bag of its occurrence, key as two
// words), or with rows (key, bag) as int32 pairs; bag_of gives the bag, and without bags the
// occurrence is its own bag.  Every load of the tile is issued first (keys, the key before each position,
// occurrence, then the bags through the occurrences; and, when FUSED, the head counts of the
// earlier tiles), then one barrier publishes the per-round wave head counts.
// FUSED: few tiles, so the block sums the head counts of the tiles before it itself, and
// the last block publishes U.
// B16: bag_of holds the 16-bit sample indices (form_keys_bags_kernel<.., true>) carried
// through the sort, in sorted order; the bag is table * batch + sample, the table taken from
// the key.  Otherwise bag_of holds 32-bit bags in occurrence order, read through the
// occurrence index.
constexpr int kFinMaxTables = 1024;
template <typename K, bool FUSED, bool B16>
__global__ __launch_bounds__(kThreads) void unique_finalize_kernel(
    const K* __restrict__ sk, const uint32_t* __restrict__ sv, const void* __restrict__ bag_of,
    int64_t n, uint64_t flip, const uint32_t* __restrict__ tile_heads, int64_t ntiles,
    int64_t* __restrict__ uniq, int32_t* __restrict__ inverse, int32_t* __restrict__ seg_offsets,
    void* __restrict__ sorted_src, bool rows, int32_t* __restrict__ num_unique,
    const int64_t* __restrict__ row_base, int num_tables, int64_t batch, int seg_bits) {
  __shared__ uint32_t wcnt[kFinRounds][4];
  __shared__ uint32_t wtile[2][4];
  __shared__ int64_t s_rb[B16 ? kFinMaxTables : 1];
  if constexpr (B16)
    for (int t = threadIdx.x; t < num_tables; t += kThreads) s_rb[t] = row_base[t];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t le = (lane == 63) ? ~0ull : ((2ull << lane) - 1ull);
  const int64_t tile = blockIdx.x;
  const int64_t t0 = tile * kFinTile;

  K key[kFinRounds];
  K prev[kFinRounds];
  uint32_t occ[kFinRounds];
  uint32_t bag[kFinRounds];
#pragma unroll
  for (int j = 0; j < kFinRounds; ++j) {
    const int64_t p = t0 + (int64_t)j * kThreads + threadIdx.x;
    const bool ok = p < n;
    key[j] = ok ? sk[p] : (K)0;
    prev[j] = (ok && p > 0) ? sk[p - 1] : (K)0;
    occ[j] = (ok && sv) ? sv[p] : ~0u;           // no payload: no inverse to scatter
  }
#pragma unroll
  for (int j = 0; j < kFinRounds; ++j) {
    const int64_t p = t0 + (int64_t)j * kThreads + threadIdx.x;
    if constexpr (B16)             // sorted with the keys: position order
      bag[j] = (p < n && bag_of) ? (uint32_t) static_cast<const uint16_t*>(bag_of)[p] : occ[j];
    else                           // occurrence order: read through the occurrence
      bag[j] = (p < n && bag_of && occ[j] < (uint64_t)n)
                   ? static_cast<const uint32_t*>(bag_of)[occ[j]] : occ[j];
  }
  uint32_t before_tile = 0, all_tiles = 0;
  if (FUSED) {
    for (int64_t t = threadIdx.x; t < ntiles; t += kThreads) {
      const uint32_t c = tile_heads[t];
      all_tiles += c;
      if (t < tile) before_tile += c;
    }
    for (int o = 32; o > 0; o >>= 1) {
      before_tile += __shfl_xor(before_tile, o, 64);
      all_tiles += __shfl_xor(all_tiles, o, 64);
    }
    if (lane == 0) {
      wtile[0][wave] = before_tile;
      wtile[1][wave] = all_tiles;
    }
  }
  uint64_t m[kFinRounds];
#pragma unroll
  for (int j = 0; j < kFinRounds; ++j) {
    const int64_t p = t0 + (int64_t)j * kThreads + threadIdx.x;
    const bool h = p < n && (p == 0 || key[j] != prev[j]);
    m[j] = __ballot(h);
    if (lane == 0) wcnt[j][wave] = (uint32_t)__popcll(m[j]);
  }
  __syncthreads();
  uint32_t base;
  if (FUSED) {
    base = wtile[0][0] + wtile[0][1] + wtile[0][2] + wtile[0][3];
    if (tile == ntiles - 1 && threadIdx.x == 0) {
      const uint32_t tot = wtile[1][0] + wtile[1][1] + wtile[1][2] + wtile[1][3];
      *num_unique = (int32_t)tot;
      if (seg_offsets) seg_offsets[tot] = (int32_t)n;
    }
  } else {
    base = tile_heads[tile];
  }
#pragma unroll
  for (int j = 0; j < kFinRounds; ++j) {
    const int64_t p = t0 + (int64_t)j * kThreads + threadIdx.x;
    uint32_t before = base;
    for (int w = 0; w < wave; ++w) before += wcnt[j][w];
    base += wcnt[j][0] + wcnt[j][1] + wcnt[j][2] + wcnt[j][3];
    if (p < n) {
      const uint32_t r = before + (uint32_t)__popcll(m[j] & le) - 1u;   // heads <= p, less one
      uint64_t kk = (uint64_t)key[j] ^ flip;
      int seg = -1;                              // table-segmented sort: (t << L) | local
      if (seg_bits) {
        seg = (int)(kk >> seg_bits) < num_tables ? (int)(kk >> seg_bits) : num_tables - 1;
        kk = (uint64_t)row_base[seg] + (kk & ((1ull << seg_bits) - 1ull));
      }
      if ((m[j] >> lane) & 1ull) {
        uniq[r] = (int64_t)kk;
        if (seg_offsets) seg_offsets[r] = (int32_t)p;
      }
      if (inverse && occ[j] < (uint64_t)n) inverse[occ[j]] = (int32_t)r;
      if (sorted_src) {
        uint32_t bg = bag[j];
        if constexpr (B16) {
          int lo = seg, hi = seg;                // the table: from the key, else the last one
          if (seg < 0) {                         // whose first row is <= the key
            lo = 0;
            hi = num_tables - 1;
          }
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((uint64_t)s_rb[mid] <= kk) lo = mid; else hi = mid - 1;
          }
          bg += (uint32_t)((int64_t)lo * batch);
        }
        if (rows)
          static_cast<int2*>(sorted_src)[p] = make_int2((int32_t)kk, (int32_t)bg);
        else
          static_cast<int4*>(sorted_src)[p] =
              make_int4((int32_t)r, (int32_t)bg, (int32_t)kk, (int32_t)(kk >> 32));
      }
    }
  }
}

__global__ void unique_empty_kernel(int32_t* num_unique, int32_t* seg_offsets) {
  if (threadIdx.x == 0) {
    *num_unique = 0;
    if (seg_offsets) seg_offsets[0] = 0;
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct UniqueWs {
  void* keys_a;
  void* keys_b;
  uint32_t* vals_a;
  uint32_t* vals_b;
  uint32_t* bags_a;           // bag of each occurrence, occurrence order (or 16-bit ones)
  uint16_t* bags16_b;         // the 16-bit sample indices' second buffer
  uint32_t* hist;
  uint32_t* totals;
  uint32_t* tile_heads;
  SegBlock* blk;              // the table-segmented sort's block map
  size_t bytes;
};

UniqueWs carve(void* base, int64_t n) {
  UniqueWs w{};
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t sz) {
    char* p = b ? b + off : nullptr;
    off += align256(sz);
    return p;
  };
  w.keys_a = take(sizeof(uint64_t) * (size_t)n);
  w.keys_b = take(sizeof(uint64_t) * (size_t)n);
  w.vals_a = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)n));
  w.vals_b = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)n));
  w.bags_a = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)n));
  w.bags16_b = reinterpret_cast<uint16_t*>(take(sizeof(uint16_t) * (size_t)n));
  w.hist = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * kBuckets * kMaxBlocks));
  w.totals = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * kBuckets));
  w.tile_heads = reinterpret_cast<uint32_t*>(
      take(sizeof(uint32_t) * (size_t)((n + kFinTile - 1) / kFinTile + 1)));
  w.blk = reinterpret_cast<SegBlock*>(take(sizeof(SegBlock) * kMaxBlocks));
  w.bytes = off;
  return w;
}

template <typename K, int ITEMS>
void radix_pass(bool first, const K* kin, const uint32_t* vin, const uint16_t* bin, K* kout,
                uint32_t* vout, uint16_t* bout, int64_t n, int shift, int nbits,
                int64_t per_block, const SegBlock* blk, uint32_t* hist, uint32_t* totals,
                int nblocks, hipStream_t s) {
  const int ld = (nblocks + 3) & ~3;
  radix_upsweep_kernel<K><<<nblocks, kThreads, 0, s>>>(kin, n, shift, nbits, per_block, blk,
                                                       hist, ld);
  const bool fused = nblocks <= kFusedScanBlocks && !blk;
  if (!fused) radix_scan_kernel<<<kBuckets, kThreads, 0, s>>>(hist, nblocks, ld, totals);
#define CTR_DS(I, FU, B, V)                                                                \
  radix_downsweep_kernel<K, ITEMS, I, FU, B, V><<<nblocks, kThreads, 0, s>>>(              \
      kin, vin, bin, kout, vout, bout, n, shift, nbits, per_block, blk, hist, totals, nblocks, \
      ld)
#define CTR_DS2(I, FU)                                              \
  if (!vout) CTR_DS(I, FU, true, false);                            \
  else if (bin) CTR_DS(I, FU, true, true);                          \
  else CTR_DS(I, FU, false, true)
  if (first) {
    if (fused) { CTR_DS2(true, true); } else { CTR_DS2(true, false); }
  } else {
    if (fused) { CTR_DS2(false, true); } else { CTR_DS2(false, false); }
  }
#undef CTR_DS2
#undef CTR_DS
}

// seg: the table-segmented sort (key_bits = the local bits): blocks are cut per table by
// seg_blocks_kernel into `blk`, at most one partial block per table.
struct SegPlan {
  const int64_t* offsets;
  int64_t batch;
  int num_tables;
  SegBlock* blk;
};

// bags_a/bags_b (may be null): the 16-bit sample indices, in occurrence order in bags_a,
// carried along; *sb receives the buffer that holds them in sorted order.  vbuf0 == null:
// no occurrence payload (bags_a is then required), *sv receives null.
template <typename K, int ITEMS>
void radix_sort(int key_bits, K* keys_a, K* keys_b, uint32_t* vbuf0, uint32_t* vbuf1,
                uint16_t* bags_a, uint16_t* bags_b, int64_t n, uint32_t* hist, uint32_t* totals,
                const K** sk, const uint32_t** sv, const uint16_t** sb, const SegPlan* seg,
                hipStream_t s) {
  constexpr int kT = kThreads * ITEMS;
  const int64_t ntiles = (n + kT - 1) / kT;
  int nblocks, spare = seg ? seg->num_tables : 0;   // a partial block per table at most
  int64_t per_block;
  {
    const int64_t avail = kMaxBlocks - spare;
    int64_t nb = ntiles < avail ? ntiles : avail;
    const int64_t tiles_per_block = (ntiles + nb - 1) / nb;
    nb = (ntiles + tiles_per_block - 1) / tiles_per_block;
    per_block = tiles_per_block * kT;
    nblocks = (int)(nb + spare);
  }
  const SegBlock* blk = nullptr;
  if (seg) {
    seg_blocks_kernel<<<1, 1024, 0, s>>>(seg->offsets, seg->batch, seg->num_tables, n, per_block,
                                         nblocks, seg->blk);
    blk = seg->blk;
  }
  const int passes = (key_bits + kMaxBits - 1) / kMaxBits;
  K* kin = keys_a;
  K* kout = keys_b;
  uint32_t* vb[2] = {vbuf0, vbuf1};
  const uint32_t* vin = nullptr;
  uint16_t* bin = bags_a;
  uint16_t* bout = bags_b;
  int shift = 0;
  for (int p = 0; p < passes; ++p) {
    const int left = key_bits - shift;
    const int nbits = left / (passes - p);   // spread evenly, the wider digits last
    uint32_t* vout = vbuf0 ? vb[(passes - 1 - p) & 1] : nullptr;    // last pass -> vbuf0
    radix_pass<K, ITEMS>(p == 0, kin, vin, bin, kout, vout, bout, n, shift, nbits, per_block,
                         blk, hist, totals, nblocks, s);
    shift += nbits;
    vin = vout;
    std::swap(kin, kout);
    std::swap(bin, bout);
  }
  *sk = kin;
  *sv = vin;
  *sb = bin;
}

template <typename K>
hipError_t unique_impl(const void* ids, bool ids64, int64_t n, const int64_t* offsets,
                       int64_t batch, int32_t num_tables, const int64_t* row_base,
                       int64_t modulus, int key_bits, int seg_bits, uint64_t flip,
                       int64_t* uniq, int32_t* inverse, int32_t* num_unique, int32_t* perm,
                       int32_t* seg_offsets, void* sorted_src, bool src_rows, UniqueWs& w,
                       hipStream_t s) {
  const bool bags = offsets != nullptr && sorted_src != nullptr;
  // 16-bit sample indices for the bags when the table can be told from the key
  const bool b16 = bags && row_base != nullptr && batch <= 65536 &&
                   num_tables <= kFinMaxTables && sizeof(K) == 4 && flip == 0;
  K* keys_a = static_cast<K*>(w.keys_a);
  K* keys_b = static_cast<K*>(w.keys_b);

  // a1: keys (and bags)
  if (offsets) {
    const int64_t num_bags = (int64_t)num_tables * batch;
    const int64_t groups = (num_bags + 63) / 64;
    // about 4096 waves, but no part shorter than one 64-occurrence stretch
    int64_t parts = (4096 + groups - 1) / groups;
    const int64_t stretches = (n / (groups > 0 ? groups : 1) + 63) / 64;
    if (parts > stretches) parts = stretches;
    if (parts < 1) parts = 1;
    const int64_t blocks = (groups * parts + 3) / 4;
    if (blocks > 0) {
#define CTR_FK(I64, B)                                                                     \
  form_keys_bags_kernel<I64, K, B><<<(unsigned)blocks, kThreads, 0, s>>>(                  \
      ids, n, offsets, batch, num_bags, row_base, modulus, flip, (int)parts, seg_bits, keys_a, \
      w.bags_a)
      if (ids64) {
        if (b16) CTR_FK(true, true); else CTR_FK(true, false);
      } else {
        if (b16) CTR_FK(false, true); else CTR_FK(false, false);
      }
#undef CTR_FK
    }
  } else {
    int64_t blocks = (n + kThreads - 1) / kThreads;
    if (blocks > 8192) blocks = 8192;
    if (ids64)
      form_keys_flat_kernel<true, K><<<(unsigned)blocks, kThreads, 0, s>>>(ids, n, modulus,
                                                                           flip, keys_a);
    else
      form_keys_flat_kernel<false, K><<<(unsigned)blocks, kThreads, 0, s>>>(ids, n, modulus,
                                                                            flip, keys_a);
  }

  // a2: stable LSD radix sort of (key, occurrence) over the live key bits; values ping-pong
  // so that the last pass lands in `perm` when the caller wants it.  The bags stay in
  // occurrence order (w.bags_a) for the finalize.
  // no occurrence payload when nothing reads it: neither the inverse map nor the permutation
  // is wanted, and the bags ride along (16-bit)
  const bool payload = inverse != nullptr || perm != nullptr || !b16;
  uint32_t* vbuf0 = !payload ? nullptr : perm ? reinterpret_cast<uint32_t*>(perm) : w.vals_a;
  uint32_t* vbuf1 = perm ? w.vals_a : w.vals_b;
  const K* sk;
  const uint32_t* sv;
  const SegPlan plan{offsets, batch, num_tables, w.blk};
  const SegPlan* seg = seg_bits ? &plan : nullptr;      // sort the local bits per table
  const int sort_bits = seg_bits ? seg_bits : key_bits;
  // 16-bit sample indices ride along through the passes; 32-bit bags stay in occurrence
  // order for the finalize to read through the occurrence index
  uint16_t* b16a = b16 ? reinterpret_cast<uint16_t*>(w.bags_a) : nullptr;
  uint16_t* b16b = b16 ? w.bags16_b : nullptr;
  const uint16_t* sb16 = nullptr;
  if (n <= (1 << 20))   // small batches: shorter tiles, more blocks, shorter chains
    radix_sort<K, 4>(sort_bits, keys_a, keys_b, vbuf0, vbuf1, b16a, b16b, n, w.hist, w.totals,
                     &sk, &sv, &sb16, seg, s);
  else
    radix_sort<K, 8>(sort_bits, keys_a, keys_b, vbuf0, vbuf1, b16a, b16b, n, w.hist, w.totals,
                     &sk, &sv, &sb16, seg, s);
  const void* sb = !bags ? nullptr : b16 ? static_cast<const void*>(sb16)
                                         : static_cast<const void*>(w.bags_a);

  // finalize: heads, their scan, and the scatter of uniq / seg / inverse / sorted_src
  const int64_t ftiles = (n + kFinTile - 1) / kFinTile;
  heads_count_kernel<K><<<(unsigned)ftiles, kThreads, 0, s>>>(sk, n, w.tile_heads);
#define CTR_FIN(FU, B)                                                                     \
  unique_finalize_kernel<K, FU, B><<<(unsigned)ftiles, kThreads, 0, s>>>(                  \
      sk, sv, sb, n, flip, w.tile_heads, ftiles, uniq, inverse, seg_offsets, sorted_src,   \
      src_rows, num_unique, row_base, num_tables, batch, seg_bits)
  if (ftiles <= kFusedHeadTiles) {
    if (b16) CTR_FIN(true, true); else CTR_FIN(true, false);
  } else {
    heads_scan_kernel<<<1, 1024, 0, s>>>(w.tile_heads, ftiles, n, num_unique, seg_offsets);
    if (b16) CTR_FIN(false, true); else CTR_FIN(false, false);
  }
#undef CTR_FIN
  return hipGetLastError();
}

}  // namespace

size_t unique_workspace_bytes(int64_t n) { return carve(nullptr, n).bytes; }

hipError_t launch_unique(const void* ids, bool ids64, int64_t n, const int64_t* offsets,
                         int64_t batch, int32_t num_tables, const int64_t* row_base,
                         int64_t modulus, int key_bits, int seg_bits, bool key_signed,
                         int64_t* uniq, int32_t* inverse, int32_t* num_unique, int32_t* perm,
                         int32_t* seg_offsets, void* sorted_src, bool src_rows,
                         void* workspace, hipStream_t s) {
  if (n == 0) {
    unique_empty_kernel<<<1, 64, 0, s>>>(num_unique, seg_offsets);
    return hipGetLastError();
  }
  UniqueWs w = carve(workspace, n);
  const uint64_t flip = key_signed ? (1ull << 63) : 0ull;
  // 32-bit keys whenever the live key range fits (a quarter less sort traffic); the
  // table-segmented sort's (t << L) | local always does (the caller checked)
  if (seg_bits || (!key_signed && key_bits <= 32))
    return unique_impl<uint32_t>(ids, ids64, n, offsets, batch, num_tables, row_base, modulus,
                                 key_bits, seg_bits, flip, uniq, inverse, num_unique, perm,
                                 seg_offsets, sorted_src, src_rows, w, s);
  return unique_impl<uint64_t>(ids, ids64, n, offsets, batch, num_tables, row_base, modulus,
                               key_bits, 0, flip, uniq, inverse, num_unique, perm, seg_offsets,
                               sorted_src, src_rows, w, s);
}

}  // namespace ctr
