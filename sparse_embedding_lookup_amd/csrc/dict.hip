// dict.hip -- inference-side lookup from an exported sparse-embedding dictionary on gfx950.
//
// "How TensorNet Supercharges Sparse Feature Training on TensorFlow", "Inference
// Optimization": online inference reads a pre-exported sparse embedding dictionary, keyed by
// the raw 64-bit feature ID (no modulus).  "Tera-scale training" review, hardware-aware
// framework figure: a hierarchical GPU parameter server keeps hot parameters in GPU HBM and
// warmer ones in CPU memory.
//
// The dictionary on the GPU is an open-addressing hash table in HBM: `capacity` (a power of
// two) slots of 16 bytes {int64 key, int64 value}, empty key -1, the home slot
// splitmix64(key) mod capacity and linear probing.  A slot's 16 bytes are one vector load, so
// a probe costs one memory access.  The value packs the dictionary row (low 32 bits) with
// an HBM-cache slot + 1 (high 32 bits; 0 = not cached).  Lookup resolves every ID of a
// batch to its value (-1: not in the dictionary); the pooled gather then reads a cached row
// from the HBM cache and any other row from the full dictionary table, which may live in
// pinned host memory (read over the host link) or in HBM.
#include "ctr_internal.h"

namespace ctr {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kEmptyKey = -1;

struct Slot {
  int64_t key;
  int64_t value;
};

__device__ __forceinline__ int64_t home_slot(int64_t key, int64_t mask) {
  return (int64_t)(splitmix64_out((uint64_t)key) & (uint64_t)mask);
}

__global__ __launch_bounds__(kThreads) void dict_clear_kernel(int4* __restrict__ slots,
                                                              int64_t capacity,
                                                              int32_t* __restrict__ status) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < capacity; i += stride)
    slots[i] = make_int4(-1, -1, -1, -1);            // key -1 (empty), value -1
  if (blockIdx.x == 0 && threadIdx.x < 3) status[threadIdx.x] = 0;
}

// status[0]: keys inserted more than once (the value kept is one of theirs); status[1]:
// negative keys (skipped); status[2]: keys that found no free slot (cannot happen when
// n < capacity, every probe sequence visits every slot).
__global__ __launch_bounds__(kThreads) void dict_insert_kernel(
    const int64_t* __restrict__ keys, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ hot_slots, int64_t n, Slot* __restrict__ slots, int64_t mask,
    int32_t* __restrict__ status) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const int64_t key = keys[i];
  if (key < 0) {
    atomicAdd(&status[1], 1);
    return;
  }
  const uint32_t hs = hot_slots ? (uint32_t)(hot_slots[i] + 1) : 0u;
  const int64_t value = (int64_t)(((uint64_t)hs << 32) | (uint32_t)rows[i]);
  int64_t h = home_slot(key, mask);
  for (int64_t probe = 0; probe <= mask; ++probe) {
    unsigned long long* kp = reinterpret_cast<unsigned long long*>(&slots[h].key);
    const unsigned long long prev =
        atomicCAS(kp, (unsigned long long)kEmptyKey, (unsigned long long)key);
    if (prev == (unsigned long long)kEmptyKey) {
      slots[h].value = value;
      return;
    }
    if (prev == (unsigned long long)key) {
      atomicAdd(&status[0], 1);
      return;
    }
    h = (h + 1) & mask;
  }
  atomicAdd(&status[2], 1);
}

// values[i] = the slot value of ids[i], or -1 when the ID is not in the table (or negative).
// The probe stops at the key or at an empty slot, and after `capacity` probes at most.
__global__ __launch_bounds__(kThreads) void dict_lookup_kernel(const int64_t* __restrict__ ids,
                                                               int64_t n,
                                                               const int4* __restrict__ slots,
                                                               int64_t mask,
                                                               int64_t* __restrict__ values) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const int64_t key = ids[i];
  int64_t v = -1;
  if (key >= 0) {
    int64_t h = home_slot(key, mask);
    for (int64_t probe = 0; probe <= mask; ++probe) {
      const int4 s = slots[h];
      const int64_t k = (int64_t)(((uint64_t)(uint32_t)s.y << 32) | (uint32_t)s.x);
      if (k == key) {
        v = (int64_t)(((uint64_t)(uint32_t)s.w << 32) | (uint32_t)s.z);
        break;
      }
      if (k == kEmptyKey) break;
      h = (h + 1) & mask;
    }
  }
  values[i] = v;
}

// Pooled gather over resolved values: out[b, t, :] = sum over the bag's occurrences of the
// row the value names (the HBM cache row when the value carries a slot of the cache, else
// the dictionary table row); a value of -1, or one naming a row outside the table, adds
// nothing.  The dictionary table has at least one row.  A group of G lanes owns one bag and
// keeps kU row loads in flight (kU = 1 when the bags average one ID, so that no load is
// spent on a bag's missing occurrences); rows are added in occurrence order.
template <int TY, int G, int VPL, int kU>
__global__ __launch_bounds__(kThreads) void dict_pool_kernel(
    const int64_t* __restrict__ values, int64_t nnz, const int64_t* __restrict__ offsets,
    int64_t batch, int64_t num_bags, const char* __restrict__ hot, int64_t hot_rows,
    const char* __restrict__ cold, int64_t cold_rows, int64_t row_bytes, int vecs,
    float* __restrict__ out, int64_t sb, int64_t st) {
  constexpr int E = TY != kEltF32 ? 8 : 4;
  const int lane = threadIdx.x & (G - 1);
  const int64_t bag = (int64_t)blockIdx.x * (kThreads / G) + threadIdx.x / G;
  if (bag >= num_bags) return;
  const int64_t o0 = clamp64(offsets[bag], 0, nnz);
  const int64_t o1 = clamp64(offsets[bag + 1], o0, nnz);
  float acc[VPL][E];
#pragma unroll
  for (int a = 0; a < VPL; ++a)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[a][e] = 0.f;
  for (int64_t k0 = o0; k0 < o1; k0 += kU) {
    uint4 rv[kU][VPL];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t k = k0 + u;
      const int64_t vk = values[k < o1 ? k : o1 - 1];          // o1 > o0 >= 0 here
      const int64_t v = k < o1 ? vk : -1;
      const uint32_t hs = (uint32_t)((uint64_t)v >> 32);
      const int64_t row = (int64_t)(uint32_t)v;
      // every lane loads from a valid row (row 0 of the table stands in for a value that
      // names nothing) and keeps the load only when the value is valid, so the loads of all
      // kU occurrences issue together.  The table is authoritative: a row whose cache slot
      // is outside the cache (or with no cache) is read from the table.
      const bool in_hot = v >= 0 && hs != 0u && (int64_t)hs - 1 < hot_rows;
      const bool in_cold = v >= 0 && !in_hot && row < cold_rows;
      const char* src = in_hot ? hot + ((int64_t)hs - 1) * row_bytes
                               : cold + (in_cold ? row : 0) * row_bytes;
      const bool keep = in_hot || in_cold;
#pragma unroll
      for (int a = 0; a < VPL; ++a) {
        const int vi = a * G + lane;
        if (vi < vecs) {
          const uint4 x = *reinterpret_cast<const uint4*>(src + (int64_t)vi * 16);
          rv[u][a] = keep ? x : make_uint4(0u, 0u, 0u, 0u);
        } else {
          rv[u][a] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (k0 + u >= o1) break;
#pragma unroll
      for (int a = 0; a < VPL; ++a) {
        if constexpr (TY != kEltF32) {
          acc[a][0] += half_lo<TY>(rv[u][a].x); acc[a][1] += half_hi<TY>(rv[u][a].x);
          acc[a][2] += half_lo<TY>(rv[u][a].y); acc[a][3] += half_hi<TY>(rv[u][a].y);
          acc[a][4 % E] += half_lo<TY>(rv[u][a].z); acc[a][5 % E] += half_hi<TY>(rv[u][a].z);
          acc[a][6 % E] += half_lo<TY>(rv[u][a].w); acc[a][7 % E] += half_hi<TY>(rv[u][a].w);
        } else {
          acc[a][0] += __uint_as_float(rv[u][a].x); acc[a][1] += __uint_as_float(rv[u][a].y);
          acc[a][2] += __uint_as_float(rv[u][a].z); acc[a][3] += __uint_as_float(rv[u][a].w);
        }
      }
    }
  }
  const int64_t t = bag / batch, b = bag - t * batch;
  float* o = out + b * sb + t * st;
#pragma unroll
  for (int a = 0; a < VPL; ++a) {
    const int vi = a * G + lane;
    if (vi < vecs) {
      float4* p = reinterpret_cast<float4*>(o + (int64_t)vi * E);
      p[0] = make_float4(acc[a][0], acc[a][1], acc[a][2], acc[a][3]);
      if (E == 8) p[1] = make_float4(acc[a][4 % E], acc[a][5 % E], acc[a][6 % E], acc[a][7 % E]);
    }
  }
}

}  // namespace

hipError_t launch_dict_build(const int64_t* keys, const int32_t* rows, const int32_t* hot_slots,
                             int64_t n, void* slots, int64_t capacity, int32_t* status,
                             hipStream_t s) {
  int64_t cb = (capacity + kThreads - 1) / kThreads;
  if (cb > 65536) cb = 65536;
  dict_clear_kernel<<<(unsigned)cb, kThreads, 0, s>>>(static_cast<int4*>(slots), capacity,
                                                      status);
  if (n > 0)
    dict_insert_kernel<<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, s>>>(
        keys, rows, hot_slots, n, static_cast<Slot*>(slots), capacity - 1, status);
  return hipGetLastError();
}

hipError_t launch_dict_lookup(const int64_t* ids, int64_t n, const void* slots,
                              int64_t capacity, int64_t* values, hipStream_t s) {
  if (n == 0) return hipSuccess;
  dict_lookup_kernel<<<(unsigned)((n + kThreads - 1) / kThreads), kThreads, 0, s>>>(
      ids, n, static_cast<const int4*>(slots), capacity - 1, values);
  return hipGetLastError();
}

hipError_t launch_dict_pool(const int64_t* values, int64_t nnz, const int64_t* offsets,
                            int64_t batch, int32_t num_tables, const void* hot,
                            int64_t hot_rows, const void* cold, int64_t cold_rows, int elt,
                            int dim, float* out, int64_t sb, int64_t st, hipStream_t s) {
  const int64_t num_bags = (int64_t)num_tables * batch;
  if (num_bags == 0) return hipSuccess;
  const int E = elt != kEltF32 ? 8 : 4;
  const int vecs = dim / E;
  const RowGeom rg = row_geom(vecs);
  const int64_t row_bytes = (int64_t)dim * (elt != kEltF32 ? 2 : 4);
  const char* hb = static_cast<const char*>(hot);
  const char* cb = static_cast<const char*>(cold);
  const bool single = nnz <= num_bags + num_bags / 2;     // about one ID per bag
#define CTR_DICT_POOL_U(G_, VPL_, U_)                                                    \
  do {                                                                                   \
    const int64_t blocks = (num_bags + (kThreads / (G_)) - 1) / (kThreads / (G_));       \
    if (elt == kEltF16)                                                                  \
      dict_pool_kernel<kEltF16, G_, VPL_, U_><<<(unsigned)blocks, kThreads, 0, s>>>(     \
          values, nnz, offsets, batch, num_bags, hb, hot_rows, cb, cold_rows, row_bytes, \
          vecs, out, sb, st);                                                            \
    else if (elt == kEltBF16)                                                            \
      dict_pool_kernel<kEltBF16, G_, VPL_, U_><<<(unsigned)blocks, kThreads, 0, s>>>(    \
          values, nnz, offsets, batch, num_bags, hb, hot_rows, cb, cold_rows, row_bytes, \
          vecs, out, sb, st);                                                            \
    else                                                                                 \
      dict_pool_kernel<kEltF32, G_, VPL_, U_><<<(unsigned)blocks, kThreads, 0, s>>>(     \
          values, nnz, offsets, batch, num_bags, hb, hot_rows, cb, cold_rows, row_bytes, \
          vecs, out, sb, st);                                                            \
  } while (0)
#define CTR_DICT_POOL(G_, VPL_)                              \
  do {                                                       \
    if (single) CTR_DICT_POOL_U(G_, VPL_, 1);                \
    else CTR_DICT_POOL_U(G_, VPL_, 8);                       \
  } while (0)
  switch (rg.G) {
    case 1: CTR_DICT_POOL(1, 1); break;
    case 2: CTR_DICT_POOL(2, 1); break;
    case 4: CTR_DICT_POOL(4, 1); break;
    case 8: CTR_DICT_POOL(8, 1); break;
    case 16: CTR_DICT_POOL(16, 1); break;
    case 32: CTR_DICT_POOL(32, 1); break;
    default:
      if (rg.VPL == 1) CTR_DICT_POOL(64, 1);
      else if (rg.VPL == 2) CTR_DICT_POOL(64, 2);
      else CTR_DICT_POOL(64, 4);
      break;
  }
#undef CTR_DICT_POOL
#undef CTR_DICT_POOL_U
  return hipGetLastError();
}

}  // namespace ctr
