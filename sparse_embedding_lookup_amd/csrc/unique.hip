// unique.hip -- batch ID deduplication on gfx950: key formation, a stable LSD radix sort
// over only the live key bits, and the unique / inverse / segment finalize.
//
// Method: "How TensorNet Supercharges Sparse Feature Training on TensorFlow", section
// "Core Optimizations": collect the batch's IDs, sort them and give each distinct ID a
// contiguous index.  The sort is ours: reduce-then-scan LSD radix with 8-bit digits.
//   upsweep   each block counts digits of its contiguous range (wave-aggregated counts)
//   scan      one block per digit scans that digit's per-block counts
//   downsweep each block ranks its tiles stably with wave64 ballot "multisplit"
//             (eight ballots give the mask of lanes holding the same digit), stages the
//             tile in LDS in digit order and writes it out in runs per digit.
// No inter-block waiting anywhere: every kernel only reads what earlier launches wrote.
#include "ctr_internal.h"

namespace ctr {
namespace {

constexpr int kThreads = 256;                 // 4 waves
constexpr int kItems = 8;                     // keys per thread per tile
constexpr int kTile = kThreads * kItems;      // 2048 keys per tile
constexpr int kBuckets = 256;                 // 8-bit digits
constexpr int kMaxBlocks = 1024;              // radix blocks (ranges) per pass
constexpr int kFinTile = 2048;                // positions per finalize block
constexpr int kMaxTablesLds = 4096;

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

// --------------------------------------------------------------------------- a1: keys
// key = row_base[t] + (modulus ? floor_mod(id, modulus) : id), XOR `flip` to make the
// signed order an unsigned one when the full 64-bit range is sorted.
template <bool ID64>
__global__ __launch_bounds__(kThreads) void form_keys_kernel(
    const void* __restrict__ ids, int64_t n, const int64_t* __restrict__ offsets, int64_t batch,
    int32_t num_tables, const int64_t* __restrict__ row_base, int64_t modulus, uint64_t flip,
    uint64_t* __restrict__ keys) {
  __shared__ int64_t tb[kMaxTablesLds + 1];
  const bool tables = row_base != nullptr;
  if (tables) {
    for (int t = threadIdx.x; t <= num_tables; t += kThreads)
      tb[t] = offsets[(int64_t)t * batch];
    __syncthreads();
  }
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    int64_t id = ID64 ? static_cast<const int64_t*>(ids)[i]
                      : (int64_t) static_cast<const int32_t*>(ids)[i];
    if (modulus > 0) {
      id %= modulus;
      if (id < 0) id += modulus;
    }
    int64_t key = id;
    if (tables) {
      int lo = 0, hi = num_tables - 1;      // last t with tb[t] <= i
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tb[mid] <= i) lo = mid; else hi = mid - 1;
      }
      key += row_base[lo];
    }
    keys[i] = (uint64_t)key ^ flip;
  }
}

// --------------------------------------------------------------------------- upsweep
__global__ __launch_bounds__(kThreads) void radix_upsweep_kernel(
    const uint64_t* __restrict__ keys, int64_t n, int shift, int nbits, int64_t per_block,
    uint32_t* __restrict__ hist, int nblocks) {
  __shared__ uint32_t cnt[4][kBuckets];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * kBuckets; i += kThreads) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const uint32_t mask = (1u << nbits) - 1u;
  const int64_t beg = (int64_t)blockIdx.x * per_block;
  const int64_t end = beg + per_block < n ? beg + per_block : n;
  for (int64_t base = beg; base < end; base += kThreads) {
    const int64_t e = base + threadIdx.x;
    const bool valid = e < end;
    const uint32_t d = valid ? (uint32_t)(keys[e] >> shift) & mask : 0u;
    const uint64_t active = __ballot(valid);
    const uint64_t m = match_digit(d, nbits, active);
    if (valid && (m & lanemask_lt()) == 0) cnt[wave][d] += (uint32_t)__popcll(m);
    (void)lane;
  }
  __syncthreads();
  for (int d = threadIdx.x; d < kBuckets; d += kThreads)
    hist[(int64_t)d * nblocks + blockIdx.x] = cnt[0][d] + cnt[1][d] + cnt[2][d] + cnt[3][d];
}

// --------------------------------------------------------------------------- scan
// Block d: exclusive scan of hist[d][0..nblocks) in place, totals[d] = row sum.
__global__ __launch_bounds__(kThreads) void radix_scan_kernel(uint32_t* __restrict__ hist,
                                                              int nblocks,
                                                              uint32_t* __restrict__ totals) {
  __shared__ uint32_t tmp[4];
  uint32_t* row = hist + (int64_t)blockIdx.x * nblocks;
  const int per = (nblocks + kThreads - 1) / kThreads;   // <= 4
  const int b0 = threadIdx.x * per;
  uint32_t local[4] = {0, 0, 0, 0};
  uint32_t sum = 0;
  for (int j = 0; j < per; ++j) {
    const int k = b0 + j;
    local[j] = k < nblocks ? row[k] : 0u;
    sum += local[j];
  }
  uint32_t total;
  uint32_t run = block_excl_scan_256(sum, tmp, &total);
  for (int j = 0; j < per; ++j) {
    const int k = b0 + j;
    if (k < nblocks) row[k] = run;
    run += local[j];
  }
  if (threadIdx.x == 0) totals[blockIdx.x] = total;
}

// --------------------------------------------------------------------------- downsweep
struct DownsweepSmem {
  uint64_t keys[kTile];
  uint32_t vals[kTile];
  uint32_t wcnt[4][kBuckets];
  uint32_t run[kBuckets];
  uint32_t tstart[kBuckets];
  uint32_t tcount[kBuckets];
  uint32_t tmp[4];
};

template <bool IDENTITY>
__global__ __launch_bounds__(kThreads) void radix_downsweep_kernel(
    const uint64_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in,
    uint64_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out, int64_t n, int shift,
    int nbits, int64_t per_block, const uint32_t* __restrict__ hist,
    const uint32_t* __restrict__ totals, int nblocks) {
  __shared__ DownsweepSmem sm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t mask = (1u << nbits) - 1u;

  // Global start of each digit for this block: digits before it, then blocks before it.
  {
    const uint32_t tot = totals[threadIdx.x];
    uint32_t all;
    const uint32_t excl = block_excl_scan_256(tot, sm.tmp, &all);
    sm.run[threadIdx.x] = excl + hist[(int64_t)threadIdx.x * nblocks + blockIdx.x];
  }
  __syncthreads();

  const int64_t beg = (int64_t)blockIdx.x * per_block;
  const int64_t end = beg + per_block < n ? beg + per_block : n;
  const uint64_t lt = lanemask_lt();

  for (int64_t tile = beg; tile < end; tile += kTile) {
    uint64_t key[kItems];
    uint32_t val[kItems];
    uint32_t rank[kItems];
    bool valid[kItems];
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
      const int64_t e = tile + (int64_t)wave * 64 * kItems + k * 64 + lane;
      valid[k] = e < end;
      key[k] = valid[k] ? keys_in[e] : 0ull;
      val[k] = valid[k] ? (IDENTITY ? (uint32_t)e : vals_in[e]) : 0u;
    }
    for (int d = lane; d < kBuckets; d += 64) sm.wcnt[wave][d] = 0;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
      const uint32_t d = (uint32_t)(key[k] >> shift) & mask;
      const uint64_t active = __ballot(valid[k]);
      const uint64_t m = match_digit(d, nbits, active);
      const uint32_t r = (uint32_t)__popcll(m & lt);
      uint32_t pre = 0;
      if (valid[k]) pre = sm.wcnt[wave][d];
      __builtin_amdgcn_wave_barrier();
      if (valid[k] && r == 0) sm.wcnt[wave][d] = pre + (uint32_t)__popcll(m);
      __builtin_amdgcn_wave_barrier();
      rank[k] = pre + r;
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
    for (int k = 0; k < kItems; ++k) {
      if (valid[k]) {
        const uint32_t d = (uint32_t)(key[k] >> shift) & mask;
        const uint32_t pos = sm.tstart[d] + sm.wcnt[wave][d] + rank[k];
        sm.keys[pos] = key[k];
        sm.vals[pos] = val[k];
      }
    }
    __syncthreads();
    const int tile_n = (int)((end - tile) < kTile ? (end - tile) : kTile);
    for (int q = threadIdx.x; q < tile_n; q += kThreads) {
      const uint64_t kk = sm.keys[q];
      const uint32_t d = (uint32_t)(kk >> shift) & mask;
      const uint32_t o = sm.run[d] + (uint32_t)q - sm.tstart[d];
      keys_out[o] = kk;
      vals_out[o] = sm.vals[q];
    }
    __syncthreads();
    sm.run[threadIdx.x] += sm.tcount[threadIdx.x];
    __syncthreads();
  }
}

// --------------------------------------------------------------------------- finalize
__global__ __launch_bounds__(kThreads) void heads_count_kernel(const uint64_t* __restrict__ sk,
                                                               int64_t n,
                                                               uint32_t* __restrict__ tile_heads) {
  __shared__ uint32_t tmp[4];
  const int64_t t0 = (int64_t)blockIdx.x * kFinTile;
  uint32_t c = 0;
  for (int j = 0; j < kFinTile / kThreads; ++j) {
    const int64_t p = t0 + (int64_t)j * kThreads + threadIdx.x;
    if (p < n) c += (p == 0 || sk[p] != sk[p - 1]) ? 1u : 0u;
  }
  uint32_t total;
  block_excl_scan_256(c, tmp, &total);
  if (threadIdx.x == 0) tile_heads[blockIdx.x] = total;
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

__global__ __launch_bounds__(kThreads) void unique_finalize_kernel(
    const uint64_t* __restrict__ sk, const uint32_t* __restrict__ sv, int64_t n, uint64_t flip,
    const uint32_t* __restrict__ tile_heads, int64_t* __restrict__ uniq,
    int32_t* __restrict__ inverse, int32_t* __restrict__ seg_offsets) {
  __shared__ uint32_t tmp[4];
  constexpr int kPer = kFinTile / kThreads;     // 8 consecutive positions per thread
  const int64_t p0 = (int64_t)blockIdx.x * kFinTile + (int64_t)threadIdx.x * kPer;
  uint64_t k[kPer];
  bool head[kPer];
  uint32_t c = 0;
  uint64_t prev = (p0 > 0 && p0 <= n) ? sk[p0 - 1] : 0ull;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t p = p0 + j;
    k[j] = p < n ? sk[p] : 0ull;
    head[j] = p < n && (p == 0 || k[j] != prev);
    prev = k[j];
    c += head[j] ? 1u : 0u;
  }
  uint32_t total;
  uint32_t run = tile_heads[blockIdx.x] + block_excl_scan_256(c, tmp, &total);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t p = p0 + j;
    if (p >= n) break;
    if (head[j]) ++run;
    const uint32_t r = run - 1u;
    if (head[j]) {
      uniq[r] = (int64_t)(k[j] ^ flip);
      if (seg_offsets) seg_offsets[r] = (int32_t)p;
    }
    const uint32_t occ = sv[p];
    if (occ < (uint64_t)n) inverse[occ] = (int32_t)r;
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
  uint64_t* keys_a;
  uint64_t* keys_b;
  uint32_t* vals_a;
  uint32_t* vals_b;
  uint32_t* hist;
  uint32_t* totals;
  uint32_t* tile_heads;
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
  w.keys_a = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * (size_t)n));
  w.keys_b = reinterpret_cast<uint64_t*>(take(sizeof(uint64_t) * (size_t)n));
  w.vals_a = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)n));
  w.vals_b = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)n));
  w.hist = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * kBuckets * kMaxBlocks));
  w.totals = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * kBuckets));
  w.tile_heads =
      reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)((n + kFinTile - 1) / kFinTile + 1)));
  w.bytes = off;
  return w;
}

}  // namespace

size_t unique_workspace_bytes(int64_t n, bool /*need_perm*/) { return carve(nullptr, n).bytes; }

hipError_t launch_unique(const void* ids, bool ids64, int64_t n, const int64_t* offsets,
                         int64_t batch, int32_t num_tables, const int64_t* row_base,
                         int64_t modulus, int key_bits, bool key_signed, int64_t* uniq,
                         int32_t* inverse, int32_t* num_unique, int32_t* perm,
                         int32_t* seg_offsets, void* workspace, hipStream_t s) {
  if (n == 0) {
    unique_empty_kernel<<<1, 64, 0, s>>>(num_unique, seg_offsets);
    return hipGetLastError();
  }
  UniqueWs w = carve(workspace, n);
  const uint64_t flip = key_signed ? (1ull << 63) : 0ull;

  // a1: keys
  {
    int64_t blocks = (n + kThreads - 1) / kThreads;
    if (blocks > 8192) blocks = 8192;
    if (ids64)
      form_keys_kernel<true><<<(unsigned)blocks, kThreads, 0, s>>>(
          ids, n, offsets, batch, num_tables, row_base, modulus, flip, w.keys_a);
    else
      form_keys_kernel<false><<<(unsigned)blocks, kThreads, 0, s>>>(
          ids, n, offsets, batch, num_tables, row_base, modulus, flip, w.keys_a);
  }

  // a2: stable LSD radix sort of (key, occurrence) over the live key bits
  const int64_t ntiles = (n + kTile - 1) / kTile;
  int nblocks = (int)(ntiles < kMaxBlocks ? ntiles : kMaxBlocks);
  const int64_t tiles_per_block = (ntiles + nblocks - 1) / nblocks;
  nblocks = (int)((ntiles + tiles_per_block - 1) / tiles_per_block);
  const int64_t per_block = tiles_per_block * kTile;
  const int passes = (key_bits + 7) / 8;

  uint64_t* kin = w.keys_a;
  uint64_t* kout = w.keys_b;
  // Values ping-pong so that the last pass lands in `perm` when the caller wants it.
  uint32_t* vbuf[2];
  if (perm) {
    vbuf[0] = reinterpret_cast<uint32_t*>(perm);
    vbuf[1] = w.vals_a;
  } else {
    vbuf[0] = w.vals_a;
    vbuf[1] = w.vals_b;
  }
  const uint32_t* vin = nullptr;
  for (int p = 0; p < passes; ++p) {
    const int shift = 8 * p;
    const int nbits = (key_bits - shift) < 8 ? (key_bits - shift) : 8;
    uint32_t* vout = vbuf[(passes - 1 - p) & 1];
    radix_upsweep_kernel<<<nblocks, kThreads, 0, s>>>(kin, n, shift, nbits, per_block, w.hist,
                                                      nblocks);
    radix_scan_kernel<<<kBuckets, kThreads, 0, s>>>(w.hist, nblocks, w.totals);
    if (p == 0)
      radix_downsweep_kernel<true><<<nblocks, kThreads, 0, s>>>(
          kin, nullptr, kout, vout, n, shift, nbits, per_block, w.hist, w.totals, nblocks);
    else
      radix_downsweep_kernel<false><<<nblocks, kThreads, 0, s>>>(
          kin, vin, kout, vout, n, shift, nbits, per_block, w.hist, w.totals, nblocks);
    vin = vout;
    uint64_t* t = kin;
    kin = kout;
    kout = t;
  }
  const uint64_t* sk = kin;
  const uint32_t* sv = vin;

  // finalize: heads, their scan, and the scatter of uniq / seg / inverse
  const int64_t ftiles = (n + kFinTile - 1) / kFinTile;
  heads_count_kernel<<<(unsigned)ftiles, kThreads, 0, s>>>(sk, n, w.tile_heads);
  heads_scan_kernel<<<1, 1024, 0, s>>>(w.tile_heads, ftiles, n, num_unique, seg_offsets);
  unique_finalize_kernel<<<(unsigned)ftiles, kThreads, 0, s>>>(sk, sv, n, flip, w.tile_heads,
                                                               uniq, inverse, seg_offsets);
  return hipGetLastError();
}

}  // namespace ctr
