// ctr_internal.h -- device helpers and kernel launchers shared by the libctr sources.
// Written for gfx950 (CDNA4, wave64) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ctr {

constexpr int kWave = 64;

// ----------------------------------------------------------------------------- bf16
// bf16 is the top half of a binary32; widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// binary32 -> bf16, round to nearest, ties to even (NaN stays a quiet NaN).  On gfx950 the
// conversion is the hardware v_cvt_pk_bf16_f32 under the default round-to-nearest-even mode.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float qnan() { return __uint_as_float(0x7FC00000u); }

// One splitmix64 output from `state` (Steele, Lea, Flood, "Fast splittable pseudorandom
// number generators", OOPSLA 2014): add the golden-ratio increment, then two
// xor-shift-multiply rounds and a final xor-shift.
__device__ __forceinline__ uint64_t splitmix64_out(uint64_t state) {
  uint64_t z = state + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Random bits of a stochastically rounded update drawn with `seed`, for the four columns
// c4 .. c4+3 (c4 a multiple of 4) of row key: one splitmix64 output from state
// seed ^ (key*dim + c4); column c4 + e takes bits 16e .. 16e+15.
__device__ __forceinline__ uint64_t sr_bits4(uint64_t seed, int64_t key, int64_t c4, int dim) {
  return splitmix64_out(seed ^ (uint64_t)(key * (int64_t)dim + c4));
}
__device__ __forceinline__ uint32_t sr_take(uint64_t bits4, int e) {
  return (uint32_t)(bits4 >> (16 * e)) & 0xFFFFu;
}

// binary32 -> bf16 with stochastic rounding ("DHEN" notes, 6.4 "Common Optimizations"):
// keep the top half of the pattern and add one unit in the last place (away from zero: the
// pattern is sign-magnitude) when r is below the dropped low half, i.e. with probability
// (|x| - |lo|) / (|hi| - |lo|).  Exact values and infinities are kept; the largest finite
// value rounding up gives infinity; NaN becomes a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_sr(float x, uint32_t r) {
  const uint32_t b = __float_as_uint(x);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (b >> 16) + (r < (b & 0xFFFFu) ? 1u : 0u);
}

// Sixteen bytes of a row widened to fp32: 4 floats (fp32 rows) or 8 floats (bf16 rows).
template <bool BF16>
struct Vec;
template <>
struct Vec<false> {
  static constexpr int kElems = 4;
  float v[4];
  __device__ __forceinline__ void zero() { v[0] = v[1] = v[2] = v[3] = 0.f; }
  __device__ __forceinline__ void nan() { v[0] = v[1] = v[2] = v[3] = qnan(); }
  __device__ __forceinline__ void load(const void* p) {
    float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
};
template <>
struct Vec<true> {
  static constexpr int kElems = 8;
  float v[8];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
  }
  __device__ __forceinline__ void nan() {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = qnan();
  }
  __device__ __forceinline__ void load(const void* p) {
    uint4 x = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16_lo(x.x); v[1] = bf16_hi(x.x);
    v[2] = bf16_lo(x.y); v[3] = bf16_hi(x.y);
    v[4] = bf16_lo(x.z); v[5] = bf16_hi(x.z);
    v[6] = bf16_lo(x.w); v[7] = bf16_hi(x.w);
  }
};

__device__ __forceinline__ int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// Row-group geometry: a row of `vecs` 16-byte vectors is handled by G lanes (a power of
// two, at most 64), each owning VPL vectors.
struct RowGeom {
  int G;
  int VPL;
};
inline RowGeom row_geom(int64_t vecs) {
  int G = 1;
  while (G < 64 && G < vecs) G <<= 1;
  int VPL = (int)((vecs + G - 1) / G);
  return {G, VPL};
}

// Records the thread's ctr_last_error text and returns code (capi.cpp).
int32_t set_error(int32_t code, const char* msg);

// ----------------------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Shapes are validated by the caller.

// unique.hip
size_t unique_workspace_bytes(int64_t n);
hipError_t launch_unique(const void* ids, bool ids64, int64_t n, const int64_t* offsets,
                         int64_t batch, int32_t num_tables, const int64_t* row_base,
                         int64_t modulus, int key_bits, bool key_signed, int64_t* uniq,
                         int32_t* inverse, int32_t* num_unique, int32_t* perm,
                         int32_t* seg_offsets, int4* sorted_src, void* workspace,
                         hipStream_t s);

// embbag.hip
hipError_t launch_embbag_fwd(const void* table, bool bf16, int64_t total_rows, int dim,
                             const int64_t* row_base, int32_t num_tables, const void* idx,
                             bool idx64, int64_t nnz, const int64_t* offsets, int64_t batch,
                             float* out, int64_t sb, int64_t st, hipStream_t s);
hipError_t launch_gather_rows(const void* table, bool bf16, int64_t total_rows, int dim,
                              const int64_t* rows, const int32_t* num_rows, int64_t capacity,
                              float* out, hipStream_t s);
hipError_t launch_sparse_sgd(void* table, bool bf16, int64_t total_rows, int dim,
                             const int64_t* uniq, const int32_t* num_unique, int64_t capacity,
                             const float* g, float lr, bool stochastic, uint64_t seed,
                             hipStream_t s);
hipError_t launch_init_table(void* table, bool bf16, int dim, int64_t row_begin,
                             int64_t rows, float scale, uint64_t seed, hipStream_t s);
hipError_t launch_validate_csr(const void* idx, bool idx64, int64_t nnz, const int64_t* offsets,
                               int64_t batch, int32_t num_tables, const int64_t* row_base,
                               int64_t total_rows, int32_t* bad, hipStream_t s);

// segreduce.hip
size_t embbag_bwd_workspace_bytes(int64_t nnz, int dim);
hipError_t launch_embbag_bwd(const void* grad, bool grad_bf16, int64_t sb, int64_t st,
                             const int64_t* offsets,
                             int64_t batch, int32_t num_tables, int dim, int64_t nnz,
                             const int32_t* perm, const int32_t* inverse, const int4* sorted_src,
                             const int32_t* num_unique, float* row_grads, void* table,
                             int sgd_mode, int64_t total_rows, const int64_t* uniq, float lr,
                             uint64_t seed, void* workspace, hipStream_t s);

// dict.hip
hipError_t launch_dict_build(const int64_t* keys, const int32_t* rows, const int32_t* hot_slots,
                             int64_t n, void* slots, int64_t capacity, int32_t* status,
                             hipStream_t s);
hipError_t launch_dict_lookup(const int64_t* ids, int64_t n, const void* slots,
                              int64_t capacity, int64_t* values, hipStream_t s);
hipError_t launch_dict_pool(const int64_t* values, int64_t nnz, const int64_t* offsets,
                            int64_t batch, int32_t num_tables, const void* hot,
                            int64_t hot_rows, const void* cold, int64_t cold_rows, bool bf16,
                            int dim, float* out, int64_t sb, int64_t st, hipStream_t s);

// interaction.hip
bool interaction_bf16_supported(int F, int dim, bool self);
bool interaction_f32_supported(int F, int dim, bool self);
hipError_t launch_interaction_fwd(const float* Z, int64_t batch, int F, int dim, bool bf16,
                                  bool self, float* R, int64_t r_stride, hipStream_t s);
hipError_t launch_interaction_bwd(const float* Z, const float* dR, int64_t dr_stride,
                                  int64_t batch, int F, int dim, bool bf16, bool self,
                                  bool out_bf16, void* dZ, hipStream_t s);
hipError_t launch_fm_fwd(const float* Z, int64_t batch, int F, int dim, float* out,
                         hipStream_t s);
hipError_t launch_fm_bwd(const float* Z, const float* dout, int64_t batch, int F, int dim,
                         float* dZ, hipStream_t s);

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
