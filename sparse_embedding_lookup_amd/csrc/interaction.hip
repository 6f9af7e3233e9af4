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
//     (staged in LDS), A = S tiles, B = Z column slabs, fp32 accumulation.
// Both paths are memory-bound on the 8 TB/s HBM: the arithmetic intensity is 6-14 flop/B.
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

__device__ __forceinline__ int tri_index(int i, int j) {
  return i > j ? i * (i - 1) / 2 + j : j * (j - 1) / 2 + i;
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* x) {
  u32x4 w;
  w[0] = f32_to_bf16_bits(x[0]) | (f32_to_bf16_bits(x[1]) << 16);
  w[1] = f32_to_bf16_bits(x[2]) | (f32_to_bf16_bits(x[3]) << 16);
  w[2] = f32_to_bf16_bits(x[4]) | (f32_to_bf16_bits(x[5]) << 16);
  w[3] = f32_to_bf16_bits(x[6]) | (f32_to_bf16_bits(x[7]) << 16);
  return __builtin_bit_cast(bf16x8, w);
}

// ------------------------------------------------------------------------- fp32 forward
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
  const int P = F * (F - 1) / 2;
  const int W = dim + P;
  for (int q = threadIdx.x; q < nb * W; q += kThreads) {
    const int s = q / W, e = q - s * W;
    float v;
    if (e < dim) {
      v = zs[(s * F) * ld + e];
    } else {
      const int pq = e - dim;
      const int i = tri_row(pq);
      const int j = pq - i * (i - 1) / 2;
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
__global__ __launch_bounds__(kThreads) void interaction_bwd_f32_kernel(
    const float* __restrict__ Z, const float* __restrict__ dR, int64_t dr_stride,
    int64_t batch, int F, int dim, int spb, float* __restrict__ dZ) {
  extern __shared__ float smem[];
  const int ld = dim + 1;
  const int P = F * (F - 1) / 2;
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
      if (j == i) continue;
      acc = __builtin_fmaf(pp[tri_index(i, j)], zc[j * ld], acc);
    }
    dZ[(b0 + s) * per + r] = acc;
  }
}

// ------------------------------------------------------------------------- bf16 forward
// FB: 32-row blocks covering F (F <= 32*FB); KS: dim / 16 (k-steps of 16).
template <int FB, int KS>
__global__ __launch_bounds__(kThreads) void interaction_fwd_mfma_kernel(
    const float* __restrict__ Z, int64_t batch, int F, float* __restrict__ R, int64_t r_stride) {
  constexpr int dim = KS * 16;
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (b >= batch) return;
  const float* zb = Z + b * (int64_t)F * dim;
  float* rb = R + b * r_stride;
  const int rl = lane & 31, kg = lane >> 5;

  // Operand fragments: lane holds row 32*I + rl, columns 16*s + 8*kg .. +8, as bf16.
  bf16x8 fr[FB][KS];
#pragma unroll
  for (int I = 0; I < FB; ++I) {
    const int row = 32 * I + rl;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float x[8];
      if (row < F) {
        const float4* p = reinterpret_cast<const float4*>(zb + row * dim + 16 * s + 8 * kg);
        const float4 a = p[0], c = p[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
      fr[I][s] = pack_bf16x8(x);
    }
  }
  for (int c = lane; c < dim; c += 64) rb[c] = zb[c];   // dense passthrough (exact)

#pragma unroll
  for (int I = 0; I < FB; ++I) {
#pragma unroll
    for (int J = 0; J <= I; ++J) {
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
        if (i < F && j < i) rb[dim + i * (i - 1) / 2 + j] = acc[v];
      }
    }
  }
}

// ------------------------------------------------------------------------- bf16 backward
// One wave per sample; WPB samples per block; LDS holds each sample's pair gradients.
template <int FB>
__global__ __launch_bounds__(kThreads) void interaction_bwd_mfma_kernel(
    const float* __restrict__ Z, const float* __restrict__ dR, int64_t dr_stride,
    int64_t batch, int F, int dim, int wpb, float* __restrict__ dZ) {
  constexpr int FKS = 2 * FB;             // k-steps of 16 over the padded F
  extern __shared__ float sp_all[];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int P = F * (F - 1) / 2;
  const int64_t b = (int64_t)blockIdx.x * wpb + wv;
  const bool live = wv < wpb && b < batch;
  float* sp = sp_all + wv * P;
  if (live)
    for (int q = lane; q < P; q += 64) sp[q] = dR[b * dr_stride + dim + q];
  __syncthreads();
  if (!live) return;
  const float* zb = Z + b * (int64_t)F * dim;
  const int rl = lane & 31, kg = lane >> 5;

  // A fragments: S[i = 32I + rl][j = 16s + 8kg + e]
  bf16x8 af[FB][FKS];
#pragma unroll
  for (int I = 0; I < FB; ++I) {
    const int i = 32 * I + rl;
#pragma unroll
    for (int s = 0; s < FKS; ++s) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 16 * s + 8 * kg + e;
        x[e] = (i < F && j < F && i != j) ? sp[tri_index(i, j)] : 0.f;
      }
      af[I][s] = pack_bf16x8(x);
    }
  }
  const int nblk = (dim + 31) / 32;
  for (int nb = 0; nb < nblk; ++nb) {
    const int n = 32 * nb + rl;
    const bool nvalid = n < dim;
    bf16x8 bfr[FKS];
#pragma unroll
    for (int s = 0; s < FKS; ++s) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 16 * s + 8 * kg + e;
        x[e] = (j < F && nvalid) ? zb[j * dim + n] : 0.f;
      }
      bfr[s] = pack_bf16x8(x);
    }
#pragma unroll
    for (int I = 0; I < FB; ++I) {
      f32x16 acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
      for (int s = 0; s < FKS; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[I][s], bfr[s], acc, 0, 0, 0);
      if (!nvalid) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = 32 * I + 8 * (v >> 2) + 4 * kg + (v & 3);
        if (i < F) {
          float val = acc[v];
          if (i == 0) val += dR[b * dr_stride + n];
          dZ[(b * F + i) * dim + n] = val;
        }
      }
    }
  }
}

// Samples per block of the fp32 kernels: as many as 32 KiB of LDS holds, but no more than
// keeps about 1024 blocks in flight (four per CU), so small batches still fill the chip.
int f32_spb(int64_t batch, int F, int dim, bool bwd) {
  const int per = (F * (dim + 1) + (bwd ? F * (F - 1) / 2 : 0)) * 4;
  int64_t spb = 32768 / per;
  const int64_t fill = batch / 1024;
  if (spb > fill) spb = fill;
  if (spb < 1) spb = 1;
  if (spb > 64) spb = 64;
  return (int)spb;
}

}  // namespace

bool interaction_bf16_supported(int F, int dim) {
  if (dim % 16 != 0 || F > 128) return false;
  const int FB = (F + 31) / 32, KS = dim / 16;
  if (!(KS == 1 || KS == 2 || KS == 4 || KS == 8)) return false;
  if (FB * KS > 32) return false;                       // register budget of the forward
  const int P = F * (F - 1) / 2;
  return P * 4 <= 65536;
}

bool interaction_f32_supported(int F, int dim) {
  const int per = (F * (dim + 1) + F * (F - 1) / 2) * 4;
  return per <= 65536;
}

#define CTR_FB_DISPATCH(FB_, ...)                        \
  switch (FB_) {                                         \
    case 1: { constexpr int FB = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int FB = 2; __VA_ARGS__; } break; \
    case 3: { constexpr int FB = 3; __VA_ARGS__; } break; \
    default: { constexpr int FB = 4; __VA_ARGS__; } break; \
  }

hipError_t launch_interaction_fwd(const float* Z, int64_t batch, int F, int dim, bool bf16,
                                  float* R, int64_t r_stride, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  if (!bf16) {
    const int spb = f32_spb(batch, F, dim, false);
    const size_t lds = (size_t)spb * F * (dim + 1) * sizeof(float);
    const int64_t blocks = (batch + spb - 1) / spb;
    interaction_fwd_f32_kernel<<<(unsigned)blocks, kThreads, lds, s>>>(Z, batch, F, dim, spb, R,
                                                                       r_stride);
    return hipGetLastError();
  }
  const int FB = (F + 31) / 32, KS = dim / 16;
  const int64_t blocks = (batch + 3) / 4;
  CTR_FB_DISPATCH(FB, {
    switch (KS) {
      case 1: interaction_fwd_mfma_kernel<FB, 1><<<(unsigned)blocks, kThreads, 0, s>>>(Z, batch, F, R, r_stride); break;
      case 2: interaction_fwd_mfma_kernel<FB, 2><<<(unsigned)blocks, kThreads, 0, s>>>(Z, batch, F, R, r_stride); break;
      case 4: interaction_fwd_mfma_kernel<FB, 4><<<(unsigned)blocks, kThreads, 0, s>>>(Z, batch, F, R, r_stride); break;
      default: interaction_fwd_mfma_kernel<FB, 8><<<(unsigned)blocks, kThreads, 0, s>>>(Z, batch, F, R, r_stride); break;
    }
  });
  return hipGetLastError();
}

hipError_t launch_interaction_bwd(const float* Z, const float* dR, int64_t dr_stride,
                                  int64_t batch, int F, int dim, bool bf16, float* dZ,
                                  hipStream_t s) {
  if (batch == 0) return hipSuccess;
  const int P = F * (F - 1) / 2;
  if (!bf16) {
    const int spb = f32_spb(batch, F, dim, true);
    const size_t lds = (size_t)spb * (F * (dim + 1) + P) * sizeof(float);
    const int64_t blocks = (batch + spb - 1) / spb;
    interaction_bwd_f32_kernel<<<(unsigned)blocks, kThreads, lds, s>>>(Z, dR, dr_stride, batch,
                                                                       F, dim, spb, dZ);
    return hipGetLastError();
  }
  const int FB = (F + 31) / 32;
  int wpb = P > 0 ? 65536 / (P * 4) : 4;
  if (wpb > 4) wpb = 4;
  if (wpb < 1) wpb = 1;
  const size_t lds = (size_t)wpb * (P > 0 ? P : 1) * sizeof(float);
  const int64_t blocks = (batch + wpb - 1) / wpb;
  CTR_FB_DISPATCH(FB, {
    interaction_bwd_mfma_kernel<FB><<<(unsigned)blocks, kThreads, lds, s>>>(
        Z, dR, dr_stride, batch, F, dim, wpb, dZ);
  });
  return hipGetLastError();
}

}  // namespace ctr
