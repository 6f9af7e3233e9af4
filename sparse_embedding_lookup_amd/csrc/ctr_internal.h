// ctr_internal.h -- device helpers shared by the libctr kernels (the launchers' host
// declarations are in ctr_launch.h, included at the end).  Written for gfx950 (CDNA4,
// wave64) only.
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

// Records the thread's ctr_last_error_message text and returns code (capi.cpp).
int32_t set_error(int32_t code, const char* msg);

// Records timing event `ev` (nothing when NULL) on stream s.  Under stream capture it adds an
// event-record node after the stream's current capture dependencies, which becomes their
// only one: a recorded event cannot be timed after a capture, such a node can (capi.cpp).
hipError_t record_mark(void* ev, hipStream_t s);

}  // namespace ctr

#include "ctr_launch.h"
