// interaction.hip -- the pairwise-dot interaction and its gradient on gfx950.
//
// Method: "Meta DLRM" (upskillscore.com), 02: the dot product between all pairs of
// embedding vectors and the processed dense features, concatenated with the dense
// features ("DHEN" notes, 3.1 and Solution 2: the vector (s_ij) over pairs, C(m,2) long).
// Per sample b, with Z[b] = (z_0 = dense, z_1..z_T = pooled), F = T + 1, P = F(F-1)/2:
//   R[b] = [ z_0 | <z_i, z_j> for F > i > j >= 0 in row-major strict-lower-triangle order ]
//   dZ_i = sum_{j != i} dP_(max,min) z_j  (+ dR_dense for i = 0)
//
// Two arithmetic paths:
//   fp32 (VALU): a block stages `spb` samples in LDS (rows padded by one float) and each
//     thread produces output elements with fused multiply-adds in column order.
//   bf16 (matrix cores): one wavefront per sample.  Forward: the Gram Z Z^T on
//     v_mfma_f32_32x32x16_bf16 over the lower-triangle 32x32 tiles, operands rounded to
//     bf16 nearest-even and kept in registers, fp32 accumulation, only i > j written.
//     Backward: dZ = S Z with S the symmetric zero-diagonal matrix of pair gradients
//     (staged in LDS), A = S tiles, B = Z column slabs, fp32 accumulation; dZ stored as
//     fp32, or rounded to bf16 for a bf16 backward (half the bytes its consumer re-reads).
// Both paths are memory-bound on the 8 TB/s HBM: the arithmetic intensity is 6-14 flop/B.
//
// Variants ("DHEN" notes, 3.1, Solution 2 and 3.3):
//   the pair set PS of every kernel below (a template parameter):
//   kStrict  the pairs i > j (above);
//   kSelf    the pairs i >= j, self-dots included ("all inner products for i <= j"):
//            P = F(F+1)/2 in row-major lower-triangle order (index i(i+1)/2 + j), and the
//            gradient of <z_i, z_i> is 2 z_i;
//   kGram    the whole Gram matrix Z Z^T that a DCN-style layer takes (3.3, eq. (7)):
//            P = F^2 in row-major order (index i F + j, both triangles: the dot of i > j is
//            computed once and written twice), and dZ_i = sum_j (dG_ij + dG_ji) z_j with the
//            two mirrored gradients added in binary32 first (the diagonal: 2 dG_ii).
//   FM sum: per sample the sum of all pair dots by the squared-norm identity,
//     out = 1/2 (||sum_i z_i||^2 - sum_i ||z_i||^2), O(F d) instead of O(F^2 d);
//     dZ_i = dout * (sum_j z_j - z_i).
#include "ctr_internal.h"

namespace ctr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// Row i of the strict lower triangle that holds pair index q (i(i-1)/2 <= q < i(i+1)/2).
__device__ __forceinline__ int tri_row(int q) {
  int i = (int)((1.0f + sqrtf(1.0f + 8.0f * (float)q)) * 0.5f);
  while (i * (i - 1) / 2 > q) --i;
  while ((i + 1) * i / 2 <= q) ++i;
  return i;
}

// tri_row for q < 2^20 without loops: the single-precision square root is within one unit in
// the last place, so the estimate is off by at most one row either way.
__device__ __forceinline__ int tri_row_small(int q) {
  int i = (int)((1.0f + __builtin_sqrtf(1.0f + 8.0f * (float)q)) * 0.5f);
  i -= (int)(i * (i - 1) / 2 > q);
  i += (int)((i + 1) * i / 2 <= q);
  return i;
}

// q = i F + j for q < 2^20 and F <= 4096, from a binary32 reciprocal of F: the estimate of i
// is off by at most one, corrected without branches.
__device__ __forceinline__ void divmod_small(int q, int F, float rcp, int* i, int* j) {
  int a = (int)((float)q * rcp);
  int r = q - a * F;
  a -= (int)(r < 0);
  r += r < 0 ? F : 0;
  a += (int)(r >= F);
  r -= r >= F ? F : 0;
  *i = a;
  *j = r;
}

__device__ __forceinline__ int tri_index(int i, int j) {
  return i > j ? i * (i - 1) / 2 + j : j * (j - 1) / 2 + i;
}

// Pair sets: strict (i > j), with self-dots (i >= j), or the whole Gram matrix.
constexpr int kStrict = kPairStrict, kSelf = kPairSelf, kGram = kPairGram;

// Outputs per sample after the dense slot, and the dots computed per sample (the Gram
// matrix computes the i >= j dots and writes the others as mirrors).
template <int PS>
__host__ __device__ constexpr int num_pairs(int F) {
  return PS == kGram ? F * F : PS == kSelf ? F * (F + 1) / 2 : F * (F - 1) / 2;
}
template <int PS>
__host__ __device__ constexpr int num_dots(int F) {
  return PS == kStrict ? F * (F - 1) / 2 : F * (F + 1) / 2;
}
__host__ inline int num_pairs_of(int pairs, int F) {
  return pairs == kGram ? num_pairs<kGram>(F) : pairs == kSelf ? num_pairs<kSelf>(F)
                                                              : num_pairs<kStrict>(F);
}
// Index of the dot (i, j) among the computed dots (i > j; i >= j unless strict).
template <int PS>
__device__ __forceinline__ int pair_index(int i, int j) {
  return PS != kStrict ? i * (i + 1) / 2 + j : i * (i - 1) / 2 + j;
}
template <int PS>
__device__ __forceinline__ int sym_pair_index(int i, int j) {
  return i >= j ? pair_index<PS>(i, j) : pair_index<PS>(j, i);
}
// Row and column of computed dot q.
template <int PS>
__device__ __forceinline__ void pair_of(int q, int* i, int* j) {
  const int r = PS != kStrict ? tri_row(q) - 1 : tri_row(q);
  *i = r;
  *j = q - (PS != kStrict ? r * (r + 1) / 2 : r * (r - 1) / 2);
}
// Stores the dot of (i, j) (i > j; i >= j unless strict) into a sample's output row o (the
// pair part): once, or at (i, j) and (j, i) for the Gram matrix.
template <int PS>
__device__ __forceinline__ void store_dot(float* o, int F, int i, int j, float v) {
  if constexpr (PS == kGram) {
    o[i * F + j] = v;
    if (i != j) o[j * F + i] = v;
  } else {
    o[pair_index<PS>(i, j)] = v;
  }
}
// Entry (i, j) of the symmetric gradient matrix S with dZ = S Z, from a sample's pair
// gradients g: the pair's gradient (i != j), twice the self-dot's (i == j, self set), zero
// on the strict set's diagonal; for the Gram matrix dG_ij + dG_ji in binary32.
template <int PS>
__device__ __forceinline__ float s_entry(const float* g, int F, int i, int j) {
  if constexpr (PS == kGram) return g[i * F + j] + g[j * F + i];
  if (i == j) return PS == kSelf ? 2.0f * g[pair_index<kSelf>(i, i)] : 0.0f;
  return g[sym_pair_index<PS>(i, j)];
}

// An empty asm that claims to change an offset: loads addressed through it stay where they
// are written instead of being hoisted out of a loop, which bounds register pressure.
__device__ __forceinline__ int pinned_zero() {
  int z = 0;
  asm volatile("" : "+v"(z));
  return z;
}

// Eight fp32 values rounded to bf16 (nearest-even, hardware convert) as an MFMA operand.
__device__ __forceinline__ bf16x8 pack_bf16x8(const float* x) {
  bf16x8 v = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3],
              (__bf16)x[4], (__bf16)x[5], (__bf16)x[6], (__bf16)x[7]};
  return v;
}

// ------------------------------------------------------------------------- fp32 forward
template <int PS>
__global__ __launch_bounds__(kThreads) void interaction_fwd_f32_kernel(
    const float* __restrict__ Z, int64_t batch, int F, int dim, int spb,
    float* __restrict__ R, int64_t r_stride) {
  extern __shared__ float zs[];
  const int ld = dim + 1;
  const int64_t b0 = (int64_t)blockIdx.x * spb;
  const int nb = (int)((batch - b0) < spb ? (batch - b0) : spb);
  const int per = F * dim;
  for (int q = threadIdx.x; q < nb * per; q += kThreads) {
    const int s = q / per, r = q - s * per;
    const int i = r / dim, c = r - i * dim;
    zs[(s * F + i) * ld + c] = Z[(b0 + s) * per + r];
  }
  __syncthreads();
  const int P = num_pairs<PS>(F);
  const int W = dim + P;
  for (int q = threadIdx.x; q < nb * W; q += kThreads) {
    const int s = q / W, e = q - s * W;
    float v;
    if (e < dim) {
      v = zs[(s * F) * ld + e];
    } else {
      // the Gram matrix's (i, j) and (j, i) are the same fused multiply-add chain
      // (multiplication commutes), so the two mirrors come out equal
      int i, j;
      if constexpr (PS == kGram) {
        i = (e - dim) / F;
        j = (e - dim) - i * F;
      } else {
        pair_of<PS>(e - dim, &i, &j);
      }
      const float* zi = zs + (s * F + i) * ld;
      const float* zj = zs + (s * F + j) * ld;
      float acc = 0.f;
      for (int c = 0; c < dim; ++c) acc = __builtin_fmaf(zi[c], zj[c], acc);
      v = acc;
    }
    R[(b0 + s) * r_stride + e] = v;
  }
}

// ------------------------------------------------------------------------- fp32 backward
template <int PS>
__global__ __launch_bounds__(kThreads) void interaction_bwd_f32_kernel(
    const float* __restrict__ Z, const float* __restrict__ dR, int64_t dr_stride,
    int64_t batch, int F, int dim, int spb, float* __restrict__ dZ) {
  extern __shared__ float smem[];
  const int ld = dim + 1;
  const int P = num_pairs<PS>(F);
  float* zs = smem;                       // [spb][F][ld]
  float* ps = smem + spb * F * ld;        // [spb][P]
  const int64_t b0 = (int64_t)blockIdx.x * spb;
  const int nb = (int)((batch - b0) < spb ? (batch - b0) : spb);
  const int per = F * dim;
  for (int q = threadIdx.x; q < nb * per; q += kThreads) {
    const int s = q / per, r = q - s * per;
    const int i = r / dim, c = r - i * dim;
    zs[(s * F + i) * ld + c] = Z[(b0 + s) * per + r];
  }
  for (int q = threadIdx.x; q < nb * P; q += kThreads) {
    const int s = q / P, r = q - s * P;
    ps[s * P + r] = dR[(b0 + s) * dr_stride + dim + r];
  }
  __syncthreads();
  for (int q = threadIdx.x; q < nb * per; q += kThreads) {
    const int s = q / per, r = q - s * per;
    const int i = r / dim, c = r - i * dim;
    float acc = (i == 0) ? dR[(b0 + s) * dr_stride + c] : 0.f;
    const float* zc = zs + (s * F) * ld + c;
    const float* pp = ps + s * P;
    for (int j = 0; j < F; ++j) {
      if (PS == kStrict && j == i) continue;
      acc = __builtin_fmaf(s_entry<PS>(pp, F, i, j), zc[j * ld], acc);
    }
    dZ[(b0 + s) * per + r] = acc;
  }
}

// ------------------------------------------------------------------------- fp32, lanes
// For F <= FMAX and dim = 4L (L a power of two, at most 64): a sample is L lanes, lane l
// holds columns 4l..4l+3 of all F vectors in registers (one 16-byte load each, all issued
// at once), so a one-wave block serves 64/L samples and a batch of B samples launches
// B*L/64 blocks.
constexpr int kLaneThreads = 64;

// Forward: R[b, 4l..] = z_0 slice; each pair's partial dot over the lane's 4 columns goes to
// LDS (dynamic: samples x P x (L + 1) floats), and after one barrier lane l sums pairs
// l, l + L, ... over the sample's L partials.  For FMAX = 32 (up to 496 pairs) the partials
// are summed with xor shuffles instead.
template <int FMAX, int L, int PS>
__global__ __launch_bounds__(kLaneThreads) void interaction_fwd_lanes_kernel(
    const float* __restrict__ Z, int64_t batch, int F, float* __restrict__ R, int64_t r_stride) {
  constexpr int kDim = 4 * L;
  constexpr bool kLds = FMAX <= 16;
  constexpr bool kSelfDots = PS != kStrict;
  extern __shared__ float part[];              // [64 / L][dots][L + 1] when kLds
  const int P = num_dots<PS>(F);
  const int lane = threadIdx.x % L;
  const int64_t b = (int64_t)blockIdx.x * (kLaneThreads / L) + threadIdx.x / L;
  const bool ok = b < batch;
  const float* zb = Z + (ok ? b : 0) * (int64_t)F * kDim + 4 * lane;
  float4 z[FMAX];
#pragma unroll
  for (int j = 0; j < FMAX; ++j)
    z[j] = j < F ? *reinterpret_cast<const float4*>(zb + j * kDim) : make_float4(0.f, 0.f, 0.f, 0.f);
  float* rb = R + (ok ? b : 0) * r_stride;
  if (ok) {                                  // r_stride need not keep 16-byte alignment
    rb[4 * lane] = z[0].x;
    rb[4 * lane + 1] = z[0].y;
    rb[4 * lane + 2] = z[0].z;
    rb[4 * lane + 3] = z[0].w;
  }
  const int sl = threadIdx.x / L;
  float* ps = part + (int64_t)sl * P * (L + 1);
  int p = 0;
#pragma unroll
  for (int i = kSelfDots ? 0 : 1; i < FMAX; ++i) {
#pragma unroll
    for (int j = 0; j < (kSelfDots ? i + 1 : i); ++j, ++p) {
      if (i < F) {
        float v = z[i].x * z[j].x;
        v = __builtin_fmaf(z[i].y, z[j].y, v);
        v = __builtin_fmaf(z[i].z, z[j].z, v);
        v = __builtin_fmaf(z[i].w, z[j].w, v);
        if constexpr (kLds) {
          ps[p * (L + 1) + lane] = v;
        } else {
#pragma unroll
          for (int o = L / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, L);
          if (ok && lane == p % L) store_dot<PS>(rb + kDim, F, i, j, v);
        }
      }
    }
  }
  if constexpr (kLds) {
    __syncthreads();
    for (int q = lane; q < P; q += L) {
      const float* row = ps + q * (L + 1);
      float v = 0.f;
#pragma unroll
      for (int l = 0; l < L; ++l) v += row[l];
      int i, j;
      pair_of<PS>(q, &i, &j);
      if (ok) store_dot<PS>(rb + kDim, F, i, j, v);
    }
  }
}

// Backward: dZ_i = sum_{j != i} dP(i, j) z_j (+ dR_dense for i = 0), one output slice at a
// time; the sample's pair gradients are staged in LDS and read as broadcasts.
template <int FMAX, int L, int PS>
__global__ __launch_bounds__(kLaneThreads) void interaction_bwd_lanes_kernel(
    const float* __restrict__ Z, const float* __restrict__ dR, int64_t dr_stride, int64_t batch,
    int F, float* __restrict__ dZ) {
  constexpr int kDim = 4 * L;
  constexpr int kS = kLaneThreads / L;                     // samples per block
  constexpr int kPmax = num_pairs<PS>(FMAX);
  __shared__ float dp[kS][kPmax];
  const int P = num_pairs<PS>(F);
  const int64_t b0 = (int64_t)blockIdx.x * kS;
  for (int q = threadIdx.x; q < kS * P; q += kLaneThreads) {
    const int s = q / P, r = q - s * P;
    dp[s][r] = b0 + s < batch ? dR[(b0 + s) * dr_stride + kDim + r] : 0.f;
  }
  const int lane = threadIdx.x % L, sl = threadIdx.x / L;
  const int64_t b = b0 + sl;
  const bool ok = b < batch;
  const float* zb = Z + (ok ? b : 0) * (int64_t)F * kDim + 4 * lane;
  float4 z[FMAX];
#pragma unroll
  for (int j = 0; j < FMAX; ++j)
    z[j] = j < F ? *reinterpret_cast<const float4*>(zb + j * kDim) : make_float4(0.f, 0.f, 0.f, 0.f);
  const float* drb = dR + (ok ? b : 0) * dr_stride + 4 * lane;     // any stride alignment
  const float4 dense = make_float4(drb[0], drb[1], drb[2], drb[3]);
  __syncthreads();
  float* db = dZ + (ok ? b : 0) * (int64_t)F * kDim + 4 * lane;
#pragma unroll
  for (int i = 0; i < FMAX; ++i) {
    if (i < F) {
      float4 acc = i == 0 ? dense : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int j = 0; j < FMAX; ++j) {
        if ((PS != kStrict || j != i) && j < F) {
          const float g = s_entry<PS>(dp[sl], F, i, j);
          acc.x = __builtin_fmaf(g, z[j].x, acc.x);
          acc.y = __builtin_fmaf(g, z[j].y, acc.y);
          acc.z = __builtin_fmaf(g, z[j].z, acc.z);
          acc.w = __builtin_fmaf(g, z[j].w, acc.w);
        }
      }
      if (ok) *reinterpret_cast<float4*>(db + i * kDim) = acc;
    }
  }
}

// Dispatch of the lane kernels: FMAX in {8, 16, 32}, L in {1, ..., 64}; false if the shape
// is not covered (then the LDS-staged kernels serve it).
#define CTR_LANES_L(FM, ...)                                                  \
  switch (L_) {                                                             \
    case 1: { constexpr int FMAX = FM, L = 1; __VA_ARGS__; } break;          \
    case 2: { constexpr int FMAX = FM, L = 2; __VA_ARGS__; } break;          \
    case 4: { constexpr int FMAX = FM, L = 4; __VA_ARGS__; } break;          \
    case 8: { constexpr int FMAX = FM, L = 8; __VA_ARGS__; } break;          \
    case 16: { constexpr int FMAX = FM, L = 16; __VA_ARGS__; } break;        \
    case 32: { constexpr int FMAX = FM, L = 32; __VA_ARGS__; } break;        \
    default: { constexpr int FMAX = FM, L = 64; __VA_ARGS__; } break;        \
  }
#define CTR_LANES(F_, L_, ...)                                               \
  do {                                                                      \
    if ((F_) <= 8) { CTR_LANES_L(8, __VA_ARGS__) }                           \
    else if ((F_) <= 16) { CTR_LANES_L(16, __VA_ARGS__) }                    \
    else { CTR_LANES_L(32, __VA_ARGS__) }                                    \
  } while (0)

bool lanes_shape(int F, int dim, int pairs) {
  const int L = dim / 4;
  if (!(F <= 32 && dim % 4 == 0 && L >= 1 && L <= 64 && (L & (L - 1)) == 0)) return false;
  // the Gram matrix's F^2 gradients per sample: the backward's LDS for F <= 16 only
  if (pairs == kGram && F > 16) return false;
  // the forward's LDS partials (F <= 16) must fit one block's 64 KiB
  const int P = pairs == kStrict ? F * (F - 1) / 2 : F * (F + 1) / 2;
  return F > 16 || (size_t)(kLaneThreads / L) * P * (L + 1) * sizeof(float) <= 65536;
}

// ------------------------------------------------------------------------- bf16 forward
// Operand fragment of row-block I, k-step s: lane holds row 32*I + rl, columns
// 16*s + 8*kg .. +8 of Z[b], rounded to bf16 (rows >= F are zero).  ZB: Z is held in bf16
// already (rounded the same way when it was stored): the fragment is one 16-byte load.
template <int KS, bool ZB>
__device__ __forceinline__ void load_row_block(const void* __restrict__ zbv, int F, int I,
                                               int rl, int kg, bf16x8* fr) {
  constexpr int dim = KS * 16;
  const int row = 32 * I + rl;
  const float* zb = static_cast<const float*>(zbv);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    float x[8];
    if constexpr (ZB) {
      if (row < F) {
        fr[s] = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(zbv) + row * dim +
                                                 16 * s + 8 * kg);
        continue;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    } else if (row < F) {
      const float4* p = reinterpret_cast<const float4*>(zb + row * dim + 16 * s + 8 * kg);
      const float4 a = p[0], c = p[1];
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    fr[s] = pack_bf16x8(x);
  }
}

// FB: 32-row blocks covering F (F <= 32*FB); KS: dim / 16 (k-steps of 16).  All FB row
// blocks of fragments stay in registers.
// ZB: Z in bf16 (the dense passthrough is then the bf16 vector, widened exactly).
template <int FB, int KS, int PS, bool ZB>
__global__ __launch_bounds__(kThreads) void interaction_fwd_mfma_kernel(
    const void* __restrict__ Z, int64_t batch, int F, float* __restrict__ R, int64_t r_stride) {
  constexpr int dim = KS * 16;
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (b >= batch) return;
  const int64_t zo = b * (int64_t)F * dim;
  const void* zb = ZB ? static_cast<const void*>(static_cast<const __bf16*>(Z) + zo)
                      : static_cast<const void*>(static_cast<const float*>(Z) + zo);
  float* rb = R + b * r_stride;
  const int rl = lane & 31, kg = lane >> 5;
  for (int c = lane; c < dim; c += 64)                  // dense passthrough (exact)
    rb[c] = ZB ? (float)static_cast<const __bf16*>(zb)[c] : static_cast<const float*>(zb)[c];

  // every row block of the sample in registers, all loads issued before any MFMA: each
  // block is read once (re-reading block J for every tile (I, J) left Large's forward at
  // 0.44 ms against 0.29)
  bf16x8 fr[FB][KS];
#pragma unroll
  for (int I = 0; I < FB; ++I) load_row_block<KS, ZB>(zb, F, I, rl, kg, fr[I]);
#pragma unroll
  for (int I = 0; I < FB; ++I) {
    if (32 * I >= F) break;
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      if (PS == kStrict && J == I && F - 32 * I < 2) break;  // no pair i > j inside this tile
      f32x16 acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[I][s], fr[J][s], acc, 0, 0, 0);
      // acc[v] = D[m][n], m = 8*(v/4) + 4*kg + v%4 (row, from A = block I), n = rl (from B)
      const int j = 32 * J + rl;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = 32 * I + 8 * (v >> 2) + 4 * kg + (v & 3);
        if (i < F && (PS != kStrict ? j <= i : j < i)) store_dot<PS>(rb + dim, F, i, j, acc[v]);
      }
    }
  }
}

// ------------------------------------------------------------------------- bf16 backward
// The product is taken transposed, dZ^T = Z^T S (S is symmetric), so that the matrix cores'
// operands come from where they are cheap:
// * A = Z^T: a lane holds 8 consecutive rows j of one column of Z (the K index of the
//   fragment).  Each fragment is loaded once (from an fp32 Z: 4-byte loads, 128 bytes per
//   row and half-wave; from a bf16 Z: through a wave-private LDS image of the slab, below),
//   rounded to bf16 and kept in registers for every row block of the output.
// * B = S: the symmetric pair-gradient matrix, rounded to bf16 once and written densely into
//   LDS (rows of 16 KM + 8 values, so rows 16 lanes apart sit in distinct banks) from
//   coalesced reads of the pair gradients; a fragment is one 16-byte row segment.
// A lane's accumulator then holds 4 consecutive columns of one dZ row, stored as one 8-
// (bf16) or 16-byte (fp32) vector.
// Work split: a wave per 32-column slab of one sample (NB = dim / 32 waves per sample, at
// least one), SPB samples per block, the sample's waves building its S together.  Every load
// of a sample (its Z slab and the first pair gradients) is issued before the first wait.
// KM: 16-row k-steps covering F.  OUTB: dZ stored as bf16 (nearest-even of the fp32 sum).
template <int KM>
__host__ __device__ constexpr int s_pitch() { return 16 * KM + 8; }
constexpr int kBwdChunk = 16;      // pair gradients per thread in flight at once

// Z rows 16 s + 8 kg .. + 7 of column n (clamped into dim) of one sample: no branch per load
// (a branch around each load serializes them), the row clamped into the sample; rows past F
// are zeroed when the fragments are packed.
// ZB: Z in bf16 (2-byte loads, widened exactly; the packing rounds them back unchanged).
template <int KM, int KS, bool ZB>
__device__ __forceinline__ void bwd_load_slab(const void* zb, int F, int n, int kg,
                                              float (&x)[KM][8]) {
  constexpr int dim = KS * 16;
  const int cn = n < dim ? n : dim - 1;
#pragma unroll
  for (int s = 0; s < KM; ++s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 16 * s + 8 * kg + e;
      const int at = (j < F ? j : F - 1) * dim + cn;
      x[s][e] = ZB ? (float)static_cast<const __bf16*>(zb)[at] : static_cast<const float*>(zb)[at];
    }
  }
}

// Pair gradients q0 + c NT + t (c < kBwdChunk) of one sample, as S entries in binary32: the
// gradient itself, or dG_ij + dG_ji for the Gram matrix.
template <int PS, int NT>
__device__ __forceinline__ void bwd_load_pairs(const float* g, int P, int F, float rcpF, int q0,
                                               int t, float (&v)[kBwdChunk]) {
#pragma unroll
  for (int c = 0; c < kBwdChunk; ++c) {
    const int q = q0 + c * NT + t;
    const int cq = q < P ? q : P - 1;
    if constexpr (PS == kGram) {
      int i, j;
      divmod_small(cq, F, rcpF, &i, &j);
      v[c] = g[cq] + g[j * F + i];      // the diagonal: 2 dG_ii
    } else {
      v[c] = g[cq];
    }
  }
}

// The same entries written into S (bf16, nearest-even), both triangles.
template <int PS, int NT, int KM>
__device__ __forceinline__ void bwd_write_pairs(__bf16* S, int P, int F, float rcpF, int q0,
                                                int t, const float (&v)[kBwdChunk]) {
  constexpr int pitch = s_pitch<KM>();
#pragma unroll
  for (int c = 0; c < kBwdChunk; ++c) {
    const int q = q0 + c * NT + t;
    if (q >= P) break;
    if constexpr (PS == kGram) {
      int i, j;
      divmod_small(q, F, rcpF, &i, &j);
      S[i * pitch + j] = (__bf16)v[c];
    } else {
      const int r = PS == kSelf ? tri_row_small(q) - 1 : tri_row_small(q);
      const int i = r, j = q - (PS == kSelf ? r * (r + 1) / 2 : r * (r - 1) / 2);
      const __bf16 h = (__bf16)v[c];
      if (i != j) {
        S[i * pitch + j] = h;
        S[j * pitch + i] = h;
      } else {
        // d<z_i, z_i>/dz_i = 2 z_i (doubling a bf16 value is exact)
        S[i * pitch + i] = (__bf16)(2.0f * (float)h);
      }
    }
  }
}

// At most 4 waves per SIMD as the occupancy target: aiming for more, the scheduler keeps
// registers low by waiting for each Z load before the next (40 loads one at a time).
// Z held in bf16, staged (ZM = 2): a wave reads its slab's 16 KM rows x 32 columns with one
// 16-byte load per 8 columns of a row (KM loads per lane, not 8 KM two-byte ones) into a
// wave-private LDS image with rows kStagePitch values apart (an odd multiple of 4 bytes
// over 8 rows, so the transposed reads of rows 8 apart fall in different banks), and takes
// its fragments' 8-row columns from there.
constexpr int kStagePitch = 36;

// ZM: Z in fp32 (0), in bf16 read directly (1), or in bf16 staged through LDS (2).
template <int KM, int KS, int PS, bool OUTB, int ZM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 4)))
void interaction_bwd_mfma_kernel(
    const void* __restrict__ Z, const float* __restrict__ dR, int64_t dr_stride,
    int64_t batch, int F, int spb, void* __restrict__ dZ) {
  constexpr int dim = KS * 16;
  constexpr int NB = (dim + 31) / 32;      // 32-column slabs: waves per sample
  constexpr int NT = NB * 64;              // threads per sample
  constexpr int FB = (KM + 1) / 2;         // 32-row blocks of dZ
  constexpr int pitch = s_pitch<KM>();     // bf16 per LDS row of S (an odd multiple of 8)
  extern __shared__ __align__(16) unsigned char s_raw[];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int sl = wv / NB;                  // sample within the block
  const int nb = wv - sl * NB;             // slab
  const int t = nb * 64 + lane;            // thread within the sample
  const int rl = lane & 31, kg = lane >> 5;
  const int n = 32 * nb + rl;              // column of Z (A row) of this lane
  __bf16* S = reinterpret_cast<__bf16*>(s_raw) + (size_t)sl * F * pitch;
  constexpr bool ZB = ZM != 0;
  const int P = num_pairs<PS>(F);
  const float rcpF = 1.0f / (float)F;
  const int64_t b = (int64_t)blockIdx.x * spb + sl;
  const bool live = b < batch;

  // S rows 0..F-1, columns 0..16 KM - 1 zeroed first: the strict set's diagonal and the
  // columns past F stay zero
  {
    u32x4* s4 = reinterpret_cast<u32x4*>(S);
    const int units = F * pitch / 8;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int u = t; u < units; u += NT) s4[u] = zero;
  }
  __syncthreads();

  // every load of the sample (its Z slab, then the first pair gradients) before any wait; S
  float x[KM][8] = {};
  if (live) {
    const float* g = dR + b * dr_stride + dim;
    float v[kBwdChunk];
    const int64_t zo = b * (int64_t)F * dim;
    if constexpr (ZM == 2) {
      // row r = task / 4 (clamped into the sample; rows past F are zeroed at the packing),
      // columns 32 nb + 8 (task % 4) .. + 7 (clamped into the row, as the direct loads clamp
      // their column)
      const __bf16* zb = static_cast<const __bf16*>(Z) + zo;
      const size_t soff = ((size_t)spb * F * pitch * 2 + 15) & ~(size_t)15;
      __bf16* zst = reinterpret_cast<__bf16*>(s_raw + soff) + (size_t)wv * (16 * KM * kStagePitch);
      uint4 q[KM];
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        const int task = lane + 64 * k, r = task >> 2, c = task & 3;
        const int row = r < F ? r : F - 1;
        const int col = 32 * nb + 8 * c < dim - 8 ? 32 * nb + 8 * c : dim - 8;
        q[k] = *reinterpret_cast<const uint4*>(zb + row * dim + col);
      }
      bwd_load_pairs<PS, NT>(g, P, F, rcpF, 0, t, v);
      bwd_write_pairs<PS, NT, KM>(S, P, F, rcpF, 0, t, v);
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        const int task = lane + 64 * k, r = task >> 2, c = task & 3;
        uint2* dst = reinterpret_cast<uint2*>(zst + r * kStagePitch + 8 * c);
        dst[0] = make_uint2(q[k].x, q[k].y);
        dst[1] = make_uint2(q[k].z, q[k].w);
      }
      // a wave's LDS accesses complete in order: its reads below see these writes
#pragma unroll
      for (int s2 = 0; s2 < KM; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          x[s2][e] = (float)zst[(16 * s2 + 8 * kg + e) * kStagePitch + rl];
    } else {
      bwd_load_slab<KM, KS, ZB>(ZB ? static_cast<const void*>(static_cast<const __bf16*>(Z) + zo)
                                   : static_cast<const void*>(static_cast<const float*>(Z) + zo),
                                F, n, kg, x);
      bwd_load_pairs<PS, NT>(g, P, F, rcpF, 0, t, v);
      bwd_write_pairs<PS, NT, KM>(S, P, F, rcpF, 0, t, v);
    }
    for (int q0 = kBwdChunk * NT; q0 < P; q0 += kBwdChunk * NT) {
      bwd_load_pairs<PS, NT>(g, P, F, rcpF, q0, t, v);
      bwd_write_pairs<PS, NT, KM>(S, P, F, rcpF, q0, t, v);
    }
  }
  // the A fragments, rows past F zeroed here rather than at the loads (a mask right after each
  // load would make the wave wait for it before the pair gradients' loads are issued)
  bf16x8 zf[KM];
#pragma unroll
  for (int s = 0; s < KM; ++s) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (16 * s + 8 * kg + e >= F) x[s][e] = 0.f;
    zf[s] = pack_bf16x8(x[s]);
  }
  __syncthreads();
  if (!live) return;

#pragma unroll
  for (int I = 0; I < FB; ++I) {
    if (32 * I >= F) break;
    const int i = 32 * I + rl;               // output row (B column); rows past F not stored
    const int ci = i < F ? i : F - 1;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < KM; ++s) {
      const bf16x8 sf = *reinterpret_cast<const bf16x8*>(S + ci * pitch + 16 * s + 8 * kg);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(zf[s], sf, acc, 0, 0, 0);
    }
    if (i >= F) continue;
    // acc[4 u + e] = dZ[i][32 nb + 8 u + 4 kg + e]
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c0 = 32 * nb + 8 * u + 4 * kg;
      if (c0 >= dim) continue;
      float val[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) val[e] = acc[4 * u + e];
      if (i == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] += dR[b * dr_stride + c0 + e];
      }
      const int64_t o = (b * F + i) * dim + c0;
      if constexpr (OUTB) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 w = {(__bf16)val[0], (__bf16)val[1], (__bf16)val[2], (__bf16)val[3]};
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(dZ) + o) = w;
      } else {
        const float4 w = {val[0], val[1], val[2], val[3]};
        *reinterpret_cast<float4*>(static_cast<float*>(dZ) + o) = w;
      }
    }
  }
}

// ------------------------------------------------------------------------- FM sum
// One wave per sample, four per block.  Lane c (columns c, c + 64, ...) forms column c of
// s = sum_i z_i and q = sum_i z_i^2 (loads coalesced across the lanes), and
// out = 1/2 sum_c (s_c^2 - q_c) is summed over the wave with xor shuffles.
__global__ __launch_bounds__(kThreads) void fm_fwd_kernel(const float* __restrict__ Z,
                                                          int64_t batch, int F, int dim,
                                                          float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (b >= batch) return;
  const float* zb = Z + b * (int64_t)F * dim;
  float acc = 0.f;
  for (int c = lane; c < dim; c += 64) {
    float sc = 0.f, qc = 0.f;
#pragma unroll 8
    for (int i = 0; i < F; ++i) {
      const float x = zb[(int64_t)i * dim + c];
      sc += x;
      qc = __builtin_fmaf(x, x, qc);
    }
    acc += __builtin_fmaf(sc, sc, -qc);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) out[b] = 0.5f * acc;
}

// dZ[b, i, c] = dout[b] * (s_c - z_ic): the column sum first, then each row.  FMAX > 0:
// the lane keeps its column of all F <= FMAX vectors in registers, so Z is read once;
// FMAX = 0 (larger F): the rows are read again (from L2 when it still holds them).  The
// column sum runs in the same order either way.
template <int FMAX>
__global__ __launch_bounds__(kThreads) void fm_bwd_kernel(const float* __restrict__ Z,
                                                          const float* __restrict__ dout,
                                                          int64_t batch, int F, int dim,
                                                          float* __restrict__ dZ) {
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (b >= batch) return;
  const float* zb = Z + b * (int64_t)F * dim;
  float* db = dZ + b * (int64_t)F * dim;
  const float g = dout[b];
  for (int c = lane; c < dim; c += 64) {
    float sc = 0.f;
    if constexpr (FMAX > 0) {
      // walking pointers with an opaque row stride: the row addresses are formed where they
      // are used, not hoisted out of the column loop (which kept 2 x FMAX 64-bit addresses
      // live)
      const int ld = dim + pinned_zero();
      float z[FMAX];
      const float* zp = zb + c;
#pragma unroll
      for (int i = 0; i < FMAX; ++i) {
        z[i] = i < F ? *zp : 0.f;
        zp += ld;
      }
#pragma unroll
      for (int i = 0; i < FMAX; ++i) sc += z[i];
      const int ld2 = dim + pinned_zero();
      float* dp = db + c;
#pragma unroll
      for (int i = 0; i < FMAX; ++i) {
        if (i < F) *dp = g * (sc - z[i]);
        dp += ld2;
      }
    } else {
#pragma unroll 8
      for (int i = 0; i < F; ++i) sc += zb[(int64_t)i * dim + c];
#pragma unroll 8
      for (int i = 0; i < F; ++i) db[(int64_t)i * dim + c] = g * (sc - zb[(int64_t)i * dim + c]);
    }
  }
}

// Samples per block of the fp32 kernels: as many as 32 KiB of LDS holds, but no more than
// keeps about 1024 blocks in flight (four per CU), so small batches still fill the chip.
int f32_spb(int64_t batch, int F, int dim, bool bwd, int pairs) {
  const int per = (F * (dim + 1) + (bwd ? num_pairs_of(pairs, F) : 0)) * 4;
  int64_t spb = 32768 / per;
  const int64_t fill = batch / 1024;
  if (spb > fill) spb = fill;
  if (spb < 1) spb = 1;
  if (spb > 64) spb = 64;
  return (int)spb;
}

}  // namespace

bool interaction_bf16_supported(int F, int dim, int pairs) {
  if (dim % 16 != 0 || F > 128) return false;
  const int FB = (F + 31) / 32, KS = dim / 16;
  if (!(KS == 1 || KS == 2 || KS == 4 || KS == 8)) return false;
  if (FB * KS > 32) return false;                       // register budget of the forward
  // one wave's dense bf16 gradient matrix in LDS (the backward)
  (void)pairs;
  return (size_t)F * (16 * ((F + 15) / 16) + 8) * 2 <= 65536;
}

bool interaction_f32_supported(int F, int dim, int pairs) {
  const int per = (F * (dim + 1) + num_pairs_of(pairs, F)) * 4;
  return per <= 65536;
}

#define CTR_FB_DISPATCH(FB_, ...)                        \
  switch (FB_) {                                         \
    case 1: { constexpr int FB = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int FB = 2; __VA_ARGS__; } break; \
    case 3: { constexpr int FB = 3; __VA_ARGS__; } break; \
    default: { constexpr int FB = 4; __VA_ARGS__; } break; \
  }

namespace {

// z_bf16 (strict pairs, matrix-core compute only; the caller checks): Z held in bf16.
template <int PS>
hipError_t interaction_fwd(const void* Zv, bool z_bf16, int64_t batch, int F, int dim, bool bf16,
                           float* R, int64_t r_stride, hipStream_t s) {
  if (z_bf16 && (!bf16 || PS != kStrict)) return hipErrorInvalidValue;
  if (batch == 0) return hipSuccess;
  const float* Z = static_cast<const float*>(Zv);   // fp32 Z (the paths below that take it)
  if (!bf16) {
    if (lanes_shape(F, dim, PS)) {
      const int P = num_dots<PS>(F);        // the forward's LDS partials
      const int L_ = dim / 4;
      const int64_t blocks = (batch * L_ + kLaneThreads - 1) / kLaneThreads;
      const size_t lds = F <= 16 ? (size_t)(kLaneThreads / L_) * P * (L_ + 1) * sizeof(float) : 0;
      CTR_LANES(F, L_, interaction_fwd_lanes_kernel<FMAX, L, PS><<<(unsigned)blocks, kLaneThreads, lds, s>>>(
                           Z, batch, F, R, r_stride));
      return hipGetLastError();
    }
    const int spb = f32_spb(batch, F, dim, false, PS);
    const size_t lds = (size_t)spb * F * (dim + 1) * sizeof(float);
    const int64_t blocks = (batch + spb - 1) / spb;
    interaction_fwd_f32_kernel<PS><<<(unsigned)blocks, kThreads, lds, s>>>(Z, batch, F, dim, spb,
                                                                           R, r_stride);
    return hipGetLastError();
  }
  const int FB = (F + 31) / 32, KS = dim / 16;
  const int64_t blocks = (batch + 3) / 4;
#define CTR_FWD_MFMA(ZB_)                                                                   \
  CTR_FB_DISPATCH(FB, {                                                                     \
    switch (KS) {                                                                           \
      case 1: interaction_fwd_mfma_kernel<FB, 1, PS, ZB_><<<(unsigned)blocks, kThreads, 0, s>>>(Zv, batch, F, R, r_stride); break; \
      case 2: interaction_fwd_mfma_kernel<FB, 2, PS, ZB_><<<(unsigned)blocks, kThreads, 0, s>>>(Zv, batch, F, R, r_stride); break; \
      case 4: interaction_fwd_mfma_kernel<FB, 4, PS, ZB_><<<(unsigned)blocks, kThreads, 0, s>>>(Zv, batch, F, R, r_stride); break; \
      default: interaction_fwd_mfma_kernel<FB, 8, PS, ZB_><<<(unsigned)blocks, kThreads, 0, s>>>(Zv, batch, F, R, r_stride); break; \
    }                                                                                       \
  })
  if constexpr (PS == kStrict) {
    if (z_bf16) {
      CTR_FWD_MFMA(true);
      return hipGetLastError();
    }
  }
  CTR_FWD_MFMA(false);
#undef CTR_FWD_MFMA
  return hipGetLastError();
}

template <int PS>
hipError_t interaction_bwd(const void* Zv, bool z_bf16, const float* dR, int64_t dr_stride,
                           int64_t batch, int F, int dim, bool bf16, bool out_bf16, void* dZv,
                           hipStream_t s) {
  // a bf16 Z is read by the matrix-core kernel of the strict pairs with a bf16 dZ only
  if (z_bf16 && (!bf16 || PS != kStrict || !out_bf16)) return hipErrorInvalidValue;
  if (batch == 0) return hipSuccess;
  const float* Z = static_cast<const float*>(Zv);   // fp32 Z (the paths below that take it)
  const int P = num_pairs<PS>(F);
  float* dZ = static_cast<float*>(dZv);
  if (!bf16) {
    if (lanes_shape(F, dim, PS)) {
      const int L_ = dim / 4;
      const int64_t blocks = (batch * L_ + kLaneThreads - 1) / kLaneThreads;
      if constexpr (PS == kGram) {          // F <= 16 (lanes_shape): F^2 gradients in LDS
        if (F <= 8) {
          CTR_LANES_L(8, interaction_bwd_lanes_kernel<FMAX, L, PS><<<(unsigned)blocks, kLaneThreads, 0, s>>>(
                             Z, dR, dr_stride, batch, F, dZ));
        } else {
          CTR_LANES_L(16, interaction_bwd_lanes_kernel<FMAX, L, PS><<<(unsigned)blocks, kLaneThreads, 0, s>>>(
                              Z, dR, dr_stride, batch, F, dZ));
        }
      } else {
        CTR_LANES(F, L_, interaction_bwd_lanes_kernel<FMAX, L, PS><<<(unsigned)blocks, kLaneThreads, 0, s>>>(
                             Z, dR, dr_stride, batch, F, dZ));
      }
      return hipGetLastError();
    }
    const int spb = f32_spb(batch, F, dim, true, PS);
    const size_t lds = (size_t)spb * (F * (dim + 1) + P) * sizeof(float);
    const int64_t blocks = (batch + spb - 1) / spb;
    interaction_bwd_f32_kernel<PS><<<(unsigned)blocks, kThreads, lds, s>>>(Z, dR, dr_stride,
                                                                           batch, F, dim, spb, dZ);
    return hipGetLastError();
  }
  const int KM = (F + 15) / 16;
  // a wave per 32-column slab; samples per block: as many as fit 4 waves and 64 KiB of LDS
  const int NB = (dim + 31) / 32;
  const int row_bytes = (16 * KM + 8) * (int)sizeof(__bf16);
  // a bf16 Z is staged through LDS where a sample's S and its waves' images fit 64 KiB
  const int zimg = 16 * KM * kStagePitch * (int)sizeof(__bf16);
  const bool zb = PS == kStrict && z_bf16;
  const bool staged = zb && F * row_bytes + 16 + NB * zimg <= 65536;
  int spb = 65536 / (F * row_bytes + (staged ? 16 + NB * zimg : 0));
  if (spb > 4 / NB) spb = 4 / NB;
  if (spb < 1) spb = 1;
  const size_t lds = staged ? (((size_t)spb * F * row_bytes + 15) & ~(size_t)15) +
                                  (size_t)spb * NB * zimg
                            : (size_t)spb * F * row_bytes;
  const int64_t blocks = (batch + spb - 1) / spb;
  const unsigned threads = (unsigned)(spb * NB * 64);
  const int KS = dim / 16;
  // a bf16 Z: strict pairs only (the pooled step's), with a bf16 dZ
#define CTR_BWD_MFMA_KS(KM_, KS_)                                                                  \
  do {                                                                                             \
    if (staged)                                                                                    \
      interaction_bwd_mfma_kernel<KM_, KS_, PS, true, PS == kStrict ? 2 : 0><<<(unsigned)blocks, threads, lds, s>>>( \
          Zv, dR, dr_stride, batch, F, spb, dZv);                                                  \
    else if (zb)                                                                                   \
      interaction_bwd_mfma_kernel<KM_, KS_, PS, true, PS == kStrict ? 1 : 0><<<(unsigned)blocks, threads, lds, s>>>( \
          Zv, dR, dr_stride, batch, F, spb, dZv);                                                  \
    else if (out_bf16)                                                                             \
      interaction_bwd_mfma_kernel<KM_, KS_, PS, true, 0><<<(unsigned)blocks, threads, lds, s>>>(   \
          Zv, dR, dr_stride, batch, F, spb, dZv);                                                  \
    else                                                                                           \
      interaction_bwd_mfma_kernel<KM_, KS_, PS, false, 0><<<(unsigned)blocks, threads, lds, s>>>(  \
          Zv, dR, dr_stride, batch, F, spb, dZv);                                                  \
  } while (0)
#define CTR_BWD_MFMA(KM_)                            \
  do {                                               \
    switch (KS) {                                    \
      case 1: CTR_BWD_MFMA_KS(KM_, 1); break;        \
      case 2: CTR_BWD_MFMA_KS(KM_, 2); break;        \
      case 4: CTR_BWD_MFMA_KS(KM_, 4); break;        \
      default: CTR_BWD_MFMA_KS(KM_, 8); break;       \
    }                                                \
  } while (0)
  switch (KM) {
    case 1: CTR_BWD_MFMA(1); break;
    case 2: CTR_BWD_MFMA(2); break;
    case 3: CTR_BWD_MFMA(3); break;
    case 4: CTR_BWD_MFMA(4); break;
    case 5: CTR_BWD_MFMA(5); break;
    case 6: CTR_BWD_MFMA(6); break;
    case 7: CTR_BWD_MFMA(7); break;
    default: CTR_BWD_MFMA(8); break;
  }
#undef CTR_BWD_MFMA_KS
#undef CTR_BWD_MFMA
  return hipGetLastError();
}

}  // namespace

hipError_t launch_interaction_fwd(const void* Z, bool z_bf16, int64_t batch, int F, int dim,
                                  bool bf16, int pairs, float* R, int64_t r_stride,
                                  hipStream_t s) {
  if (pairs == kGram)
    return interaction_fwd<kGram>(Z, false, batch, F, dim, bf16, R, r_stride, s);
  if (pairs == kSelf)
    return interaction_fwd<kSelf>(Z, false, batch, F, dim, bf16, R, r_stride, s);
  return interaction_fwd<kStrict>(Z, z_bf16, batch, F, dim, bf16, R, r_stride, s);
}

hipError_t launch_interaction_bwd(const void* Z, bool z_bf16, const float* dR,
                                  int64_t dr_stride, int64_t batch, int F, int dim, bool bf16,
                                  int pairs, bool out_bf16, void* dZ, hipStream_t s) {
  if (pairs == kGram)
    return interaction_bwd<kGram>(Z, false, dR, dr_stride, batch, F, dim, bf16, out_bf16, dZ, s);
  if (pairs == kSelf)
    return interaction_bwd<kSelf>(Z, false, dR, dr_stride, batch, F, dim, bf16, out_bf16, dZ, s);
  return interaction_bwd<kStrict>(Z, z_bf16, dR, dr_stride, batch, F, dim, bf16, out_bf16, dZ,
                                  s);
}

hipError_t launch_fm_fwd(const float* Z, int64_t batch, int F, int dim, float* out,
                         hipStream_t s) {
  if (batch == 0) return hipSuccess;
  const int64_t blocks = (batch + 3) / 4;
  fm_fwd_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(Z, batch, F, dim, out);
  return hipGetLastError();
}

hipError_t launch_fm_bwd(const float* Z, const float* dout, int64_t batch, int F, int dim,
                         float* dZ, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  const int64_t blocks = (batch + 3) / 4;
#define CTR_FM_BWD(FM) \
  fm_bwd_kernel<FM><<<(unsigned)blocks, kThreads, 0, s>>>(Z, dout, batch, F, dim, dZ)
  if (F <= 16) CTR_FM_BWD(16);
  else if (F <= 32) CTR_FM_BWD(32);
  else if (F <= 64) CTR_FM_BWD(64);
  else if (F <= 96) CTR_FM_BWD(96);
  else if (F <= 128) CTR_FM_BWD(128);
  else CTR_FM_BWD(0);
#undef CTR_FM_BWD
  return hipGetLastError();
}

}  // namespace ctr
