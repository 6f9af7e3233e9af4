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

// ----------------------------------------------------------------------------- binary16
// IEEE binary16 (1 sign, 5 exponent, 10 fraction bits; largest finite 65504, subnormal
// quantum 2^-24).  Widening to binary32 is exact; the narrowing below is the hardware
// conversion under the default round-to-nearest-even mode (overflow gives infinity,
// subnormals are kept).
__device__ __forceinline__ float f16_lo(uint32_t pair) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(pair & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t pair) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(pair >> 16));
}
// The empty asm pins f as the binary32 value it is: without it the compiler may fold the
// multiply or fused multiply-add that produced f into one mixed-precision instruction
// (v_fma_mixlo_f16) that rounds the exact result to binary16 once, skipping the binary32
// rounding the stored value is defined by.
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  __asm__ volatile("" : "+v"(f));
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// binary32 -> binary16 with stochastic rounding, the same rule as f32_to_bf16_sr: with lo
// the binary16 value next to x toward zero and q the binary16 spacing there, round away from
// zero iff r < 2^16 (|x| - |lo|) / q.  In the normal range 13 bits are dropped, so that
// threshold is the dropped bits times 8; below 2^-14 the spacing is 2^-24 and the fraction
// is taken in binary32 arithmetic, which is exact there.  |x| >= 2^16 (and infinity) gives
// infinity, as does rounding up from the largest finite binade; NaN gives a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_f16_sr(float x, uint32_t r) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t sign = (b >> 16) & 0x8000u;
  const uint32_t a = b & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7E00u;
  if (a >= 0x47800000u) return sign | 0x7C00u;
  uint32_t h;
  bool up;
  if (a >= 0x38800000u) {                       // 2^-14 <= |x| < 2^16
    const uint32_t m = a & 0x7FFFFFu;
    h = (((a >> 23) - 112u) << 10) | (m >> 13);
    up = r < ((m & 0x1FFFu) << 3);
  } else {                                      // binary16 subnormals and zero
    const float q = __uint_as_float(a) * 16777216.0f;    // |x| / 2^-24, exact
    const float n = __builtin_truncf(q);
    h = (uint32_t)n;
    up = (float)r < (q - n) * 65536.0f;
  }
  return sign | (h + (up ? 1u : 0u));
}

// Stored element types of a table row: binary32, bfloat16 or binary16 (the two 16-bit types
// hold 8 values per 16-byte vector, binary32 4).
enum : int { kEltF32 = 0, kEltBF16 = 1, kEltF16 = 2 };

template <int TY>
__device__ __forceinline__ float half_lo(uint32_t pair) {
  if constexpr (TY == kEltF16) return f16_lo(pair);
  else return bf16_lo(pair);
}
template <int TY>
__device__ __forceinline__ float half_hi(uint32_t pair) {
  if constexpr (TY == kEltF16) return f16_hi(pair);
  else return bf16_hi(pair);
}
// binary32 -> the 16-bit type, nearest-even (SR false) or stochastic with bits r (SR true).
template <int TY, bool SR>
__device__ __forceinline__ uint32_t to_half(float f, uint32_t r) {
  if constexpr (TY == kEltF16) return SR ? f32_to_f16_sr(f, r) : f32_to_f16_bits(f);
  else return SR ? f32_to_bf16_sr(f, r) : f32_to_bf16_bits(f);
}

// Sixteen bytes of a row widened to fp32: 4 floats (binary32 rows) or 8 floats (16-bit rows).
// TY is a kElt code (a bool selects binary32 or bfloat16).
template <int TY>
struct Vec;
template <>
struct Vec<kEltF32> {
  static constexpr int kElems = 4;
  float v[4];
  __device__ __forceinline__ void zero() { v[0] = v[1] = v[2] = v[3] = 0.f; }
  __device__ __forceinline__ void nan() { v[0] = v[1] = v[2] = v[3] = qnan(); }
  __device__ __forceinline__ void load(const void* p) {
    float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
};
template <int TY>
struct Vec {
  static_assert(TY == kEltBF16 || TY == kEltF16, "a 16-bit element type");
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
    v[0] = half_lo<TY>(x.x); v[1] = half_hi<TY>(x.x);
    v[2] = half_lo<TY>(x.y); v[3] = half_hi<TY>(x.y);
    v[4] = half_lo<TY>(x.z); v[5] = half_hi<TY>(x.z);
    v[6] = half_lo<TY>(x.w); v[7] = half_hi<TY>(x.w);
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
