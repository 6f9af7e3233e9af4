// dense.hip -- the fully connected layers on either side of the interaction and the
// logistic head with its normalized-entropy statistics, on gfx950.
//
// Method: "Meta DLRM" (upskillscore.com), 02 "Arquitetura": the continuous features go
// through a bottom MLP whose output is the dense vector of the interaction; the
// interaction's output goes through a top MLP and a sigmoid, which gives the click
// probability.  04: the MLPs are replicated (data parallel) and their parameter updates are
// applied synchronously.  "DHEN" notes, 7.1 "Setup": the loss is normalized entropy (NE),
// the mean binary cross-entropy divided by the entropy of the empirical click rate;
// Solution 17: with p = sigmoid(s), the cross-entropy of a logit s is softplus(s) - y s,
// stable for every s.
//
// One layer: Y[m, n] = act(sum_k X[m, k] W[n, k] + b[n]), act = ReLU or the identity.
// Its backward, with the SGD update of the layer's parameters fused:
//   dA = dY * [Y > 0] (ReLU) or dY;   dX = dA W (with W before the update);
//   W -= lr dA^T X;                   b -= lr sum_m dA[m, :].
// Gradients are sums over the batch rows (no 1/M), as for the embedding rows; the head's
// gradient carries the 1/M of the mean cross-entropy.
//
// GEMMs run on the matrix cores.  A 256-thread block owns a 128x128 output tile: four
// waves of 64x64, each 2x2 MFMA tiles of 32x32.  The reduction advances in k-tiles of 32
// staged through LDS, with the next k-tile's global loads in flight during the current
// one's MFMAs.  fp32 compute: v_mfma_f32_32x32x2f32 on fp32 operands; bf16 compute:
// v_mfma_f32_32x32x16_bf16 on operands rounded to bf16 nearest-even as they enter LDS.
// Both accumulate in fp32.  The weight gradient reduces over the batch: when its output
// tiles are too few to fill the chip, the reduction is split over grid.z into fp32 partials
// that a second pass sums in a fixed order before the update (deterministic, no atomics).
#include "ctr_internal.h"

#include <type_traits>

namespace ctr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kGemmThreads = 256;
constexpr int kColRows = 64;          // rows per block of the ReLU-backward / bias pass
constexpr int kHeadThreads = 1024;

enum Epilogue { kStore = 0, kBiasAct = 1, kSgd = 2, kPartial = 3 };

// C[m, n] (m < M, n < N) from A[m, k] and B[k, n] (k < K):
//   A[m, k] = AK ? A[m * lda + k] : A[k * lda + m]
//   B[k, n] = BK ? B[n * ldb + k] : B[k * ldb + n]
//   C[m, n] at C[m * ldc + n]; kPartial: slice z at C[(z * M + m) * ldc + n]
struct GemmArgs {
  const float* A;
  int64_t lda;
  const float* B;
  int64_t ldb;
  int64_t M, N, K;
  float* C;
  int64_t ldc;
  const float* bias;   // kBiasAct, nullable
  int relu;            // kBiasAct
  float lr;            // kSgd
  int64_t k_split;     // reduction length per grid.z slice, a multiple of kBK
  int64_t n_tiles;     // output tiles along n (the block index runs along n first)
  int vec_a, vec_b;    // operand 16-byte aligned with a stride that is a multiple of 4
};

// Operand P[r, k] (r < rows, k < kend): KMAJ ? P[r * ld + k] : P[k * ld + r].  Thread t
// loads 16 elements of the 128 x 32 tile at (r0, k0), four runs of 4 along the contiguous
// direction: KMAJ: rows (t >> 3) + 32 q, columns 4 (t & 7) + e; otherwise rows 4 (t & 31) + e,
// columns (t >> 5) + 8 q; slot 4 q + e.  Elements outside the operand are zero.
template <bool KMAJ>
__device__ __forceinline__ void load_tile(const float* __restrict__ P, int64_t ld,
                                          int64_t rows, int64_t kend, int64_t r0, int64_t k0,
                                          bool vec, float (&v)[16]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t r = KMAJ ? r0 + (t >> 3) + 32 * q : r0 + 4 * (t & 31);
    const int64_t k = KMAJ ? k0 + 4 * (t & 7) : k0 + (t >> 5) + 8 * q;
    const bool full = KMAJ ? (r < rows && k + 3 < kend) : (r + 3 < rows && k < kend);
    if (vec && full) {
      const float4 x = *reinterpret_cast<const float4*>(KMAJ ? P + r * ld + k : P + k * ld + r);
      v[4 * q] = x.x;
      v[4 * q + 1] = x.y;
      v[4 * q + 2] = x.z;
      v[4 * q + 3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t rr = KMAJ ? r : r + e, kk = KMAJ ? k + e : k;
        v[4 * q + e] = (rr < rows && kk < kend) ? P[KMAJ ? rr * ld + kk : kk * ld + rr] : 0.f;
      }
    }
  }
}

// The tile in LDS as [128 rows][PITCH], k contiguous, in the compute type (the conversion to
// bf16 is the nearest-even rounding of the operand).
template <bool KMAJ, typename LT, int PITCH>
__device__ __forceinline__ void store_tile(LT* __restrict__ lds, const float (&v)[16]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = KMAJ ? (t >> 3) + 32 * q : 4 * (t & 31) + e;
      const int k = KMAJ ? 4 * (t & 7) + e : (t >> 5) + 8 * q;
      lds[r * PITCH + k] = (LT)v[4 * q + e];
    }
}

template <bool BF, bool AK, bool BK, int EPI>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmArgs g) {
  using LT = typename std::conditional<BF, __bf16, float>::type;
  // bf16 rows stay 16-byte aligned for the 8-element fragment reads; fp32 rows are padded
  // by one word against bank conflicts of the column-wise fragment reads
  constexpr int PITCH = BF ? kBK + 8 : kBK + 1;
  __shared__ LT As[kBM * PITCH];
  __shared__ LT Bs[kBN * PITCH];

  const int64_t tile = blockIdx.x;
  const int64_t n0 = (tile % g.n_tiles) * kBN;
  const int64_t m0 = (tile / g.n_tiles) * kBM;
  const int64_t kb = (int64_t)blockIdx.z * g.k_split;
  const int64_t ke = g.K < kb + g.k_split ? g.K : kb + g.k_split;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = wv >> 1, wn = wv & 1, rl = lane & 31, kg = lane >> 5;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  float va[16], vb[16];
  if (kb < ke) {
    load_tile<AK>(g.A, g.lda, g.M, ke, m0, kb, g.vec_a, va);
    load_tile<BK>(g.B, g.ldb, g.N, ke, n0, kb, g.vec_b, vb);
  }
  for (int64_t k0 = kb; k0 < ke; k0 += kBK) {
    store_tile<AK, LT, PITCH>(As, va);
    store_tile<BK, LT, PITCH>(Bs, vb);
    __syncthreads();
    if (k0 + kBK < ke) {                 // next k-tile's loads overlap this tile's MFMAs
      load_tile<AK>(g.A, g.lda, g.M, ke, m0, k0 + kBK, g.vec_a, va);
      load_tile<BK>(g.B, g.ldb, g.N, ke, n0, k0 + kBK, g.vec_b, vb);
    }
    if constexpr (BF) {
      // fragment: lane holds row rl, k = 16 s + 8 kg .. +8 (A: rows m, B: rows n of Bs)
#pragma unroll
      for (int s = 0; s < kBK / 16; ++s) {
        bf16x8 a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          a[i] = *reinterpret_cast<const bf16x8*>(As + (64 * wm + 32 * i + rl) * PITCH +
                                                  16 * s + 8 * kg);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          b[j] = *reinterpret_cast<const bf16x8*>(Bs + (64 * wn + 32 * j + rl) * PITCH +
                                                  16 * s + 8 * kg);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    } else {
      // fragment: lane holds row rl, k = 2 s + kg
#pragma unroll
      for (int s = 0; s < kBK / 2; ++s) {
        float a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = As[(64 * wm + 32 * i + rl) * PITCH + 2 * s + kg];
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = Bs[(64 * wn + 32 * j + rl) * PITCH + 2 * s + kg];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // acc[i][j][v] = C[m, n]: m = 8 (v / 4) + 4 kg + v % 4 and n = rl within the 32x32 tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + 64 * wn + 32 * j + rl;
      if (n >= g.N) continue;
      float bn = 0.f;
      if constexpr (EPI == kBiasAct) bn = g.bias ? g.bias[n] : 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * kg + (v & 3);
        if (m >= g.M) continue;
        float x = acc[i][j][v];
        if constexpr (EPI == kStore) {
          g.C[m * g.ldc + n] = x;
        } else if constexpr (EPI == kBiasAct) {
          x += bn;
          if (g.relu) x = x > 0.f ? x : 0.f;
          g.C[m * g.ldc + n] = x;
        } else if constexpr (EPI == kSgd) {
          float* c = g.C + m * g.ldc + n;
          *c = __builtin_fmaf(-g.lr, x, *c);
        } else {
          g.C[((int64_t)blockIdx.z * g.M + m) * g.ldc + n] = x;
        }
      }
    }
}

// W[i] -= lr * (sum over the S slices of part[s * count + i]), slices in order.
__global__ __launch_bounds__(256) void sgd_from_partials_kernel(
    const float* __restrict__ part, int64_t count, int S, float lr, float* __restrict__ W) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  float s = 0.f;
  for (int z = 0; z < S; ++z) s += part[z * count + i];
  W[i] = __builtin_fmaf(-lr, s, W[i]);
}

// dA[m, n] = dY[m, n] * [Y[m, n] > 0] (or dY), contiguous [M, N]; colpart[chunk, n] = the
// sum of the chunk's kColRows rows of dA, over four interleaved accumulators.
template <bool DYB>
__global__ __launch_bounds__(256) void relu_bwd_kernel(
    const void* __restrict__ dY, int64_t dys, const float* __restrict__ Y, int64_t ys,
    int64_t M, int64_t N, int relu, float* __restrict__ dA, float* __restrict__ colpart) {
  // block = (column block, row chunk), column blocks fastest
  const int64_t cb = (N + 255) / 256;
  const int64_t chunk = (int64_t)blockIdx.x / cb;
  const int64_t n = ((int64_t)blockIdx.x % cb) * 256 + threadIdx.x;
  if (n >= N) return;
  const int64_t mb = chunk * kColRows;
  const int64_t me = M < mb + kColRows ? M : mb + kColRows;
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  for (int64_t m = mb; m < me; ++m) {
    float gv;
    if constexpr (DYB)
      gv = __uint_as_float((uint32_t)static_cast<const uint16_t*>(dY)[m * dys + n] << 16);
    else
      gv = static_cast<const float*>(dY)[m * dys + n];
    if (relu && !(Y[m * ys + n] > 0.f)) gv = 0.f;
    dA[m * N + n] = gv;
    s[(m - mb) & 3] += gv;
  }
  colpart[chunk * N + n] = (s[0] + s[1]) + (s[2] + s[3]);
}

// b[n] -= lr * (sum over chunks of colpart[c, n]), over eight interleaved accumulators.
__global__ __launch_bounds__(256) void bias_sgd_kernel(const float* __restrict__ colpart,
                                                       int64_t chunks, int64_t N, float lr,
                                                       float* __restrict__ b) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t c = 0; c < chunks; ++c) s[c & 7] += colpart[c * N + n];
  const float t = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
  b[n] = __builtin_fmaf(-lr, t, b[n]);
}

// The logistic head over M logits (one block): p = sigmoid(s), the cross-entropy
// ce = softplus(s) - y s computed as (max(s, 0) - y s) + log1p(exp(-|s|)), the gradient of
// the mean cross-entropy (p - y) / M, and stats = [sum ce, sum y, NE], where
// NE = (sum ce / M) / H(sum y / M) and H(q) = -(q ln q + (1 - q) ln(1 - q)) (NaN when every
// label is 0 or every label is 1).
__global__ __launch_bounds__(kHeadThreads) void logistic_ne_kernel(
    const float* __restrict__ s, int64_t ss, const float* __restrict__ y, int64_t M,
    float* __restrict__ prob, float* __restrict__ dl, int64_t dls, float* __restrict__ stats) {
  __shared__ float red_ce[kHeadThreads], red_y[kHeadThreads];
  const int t = threadIdx.x;
  const float fm = (float)M;
  float ce = 0.f, ys = 0.f;
  for (int64_t i = t; i < M; i += kHeadThreads) {
    const float x = s[i * ss], l = y[i];
    const float e = expf(-fabsf(x));
    const float p = x >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
    ce += (fmaxf(x, 0.f) - l * x) + log1pf(e);
    ys += l;
    if (prob) prob[i] = p;
    if (dl) dl[i * dls] = (p - l) / fm;
  }
  red_ce[t] = ce;
  red_y[t] = ys;
  __syncthreads();
  for (int h = kHeadThreads / 2; h > 0; h >>= 1) {
    if (t < h) {
      red_ce[t] += red_ce[t + h];
      red_y[t] += red_y[t + h];
    }
    __syncthreads();
  }
  if (t == 0) {
    const double sc = red_ce[0], sy = red_y[0];
    const double q = sy / (double)M;
    const double h = -(q * log(q) + (1.0 - q) * log(1.0 - q));
    stats[0] = (float)sc;
    stats[1] = (float)sy;
    stats[2] = (q > 0.0 && q < 1.0) ? (float)((sc / (double)M) / h) : qnan();
  }
}

bool vec_ok(const float* p, int64_t ld) {
  return ((uintptr_t)p & 15) == 0 && (ld & 3) == 0;
}

template <bool AK, bool BK, int EPI>
hipError_t launch_gemm(bool bf16, GemmArgs g, int splits, hipStream_t s) {
  g.n_tiles = (g.N + kBN - 1) / kBN;
  const int64_t tiles = g.n_tiles * ((g.M + kBM - 1) / kBM);
  if (tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)tiles, 1, (unsigned)splits);
  if (bf16)
    gemm_kernel<true, AK, BK, EPI><<<grid, kGemmThreads, 0, s>>>(g);
  else
    gemm_kernel<false, AK, BK, EPI><<<grid, kGemmThreads, 0, s>>>(g);
  return hipGetLastError();
}

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

// Slices of the weight-gradient reduction over the M batch rows: none while the output
// tiles alone give a block per compute unit, else enough for about two blocks per unit,
// each slice at least 512 rows long.  *k_split: rows per slice (a multiple of the k-tile).
int dense_wgrad_splits(int64_t M, int N, int K, int64_t* k_split) {
  const int64_t tiles = (int64_t)((N + kBM - 1) / kBM) * ((K + kBN - 1) / kBN);
  int64_t S = 1;
  if (tiles < 256) {
    S = (512 + tiles - 1) / tiles;
    const int64_t cap = M / 512 > 1 ? M / 512 : 1;
    if (S > cap) S = cap;
  }
  int64_t ks = (M + S - 1) / S;
  ks = (ks + kBK - 1) / kBK * kBK;
  if (ks < kBK) ks = kBK;
  S = (M + ks - 1) / ks;
  if (S < 1) S = 1;
  if (k_split) *k_split = ks;
  return (int)S;
}

size_t dense_bwd_workspace_bytes(int64_t M, int N, int K) {
  const int64_t chunks = (M + kColRows - 1) / kColRows;
  const int S = dense_wgrad_splits(M, N, K, nullptr);
  size_t b = round256((size_t)M * N * sizeof(float)) +
             round256((size_t)chunks * N * sizeof(float));
  if (S > 1) b += round256((size_t)S * N * K * sizeof(float));
  return b;
}

hipError_t launch_dense_fwd(const float* X, int64_t xs, int64_t M, int K, const float* W,
                            const float* b, int N, bool relu, bool bf16, float* Y, int64_t ys,
                            hipStream_t s) {
  if (M == 0) return hipSuccess;
  GemmArgs g{};
  g.A = X;
  g.lda = xs;
  g.B = W;
  g.ldb = K;
  g.M = M;
  g.N = N;
  g.K = K;
  g.C = Y;
  g.ldc = ys;
  g.bias = b;
  g.relu = relu;
  g.k_split = ((int64_t)K + kBK - 1) / kBK * kBK;
  g.vec_a = vec_ok(X, xs);
  g.vec_b = vec_ok(W, K);
  return launch_gemm<true, true, kBiasAct>(bf16, g, 1, s);
}

hipError_t launch_dense_bwd_sgd(const float* X, int64_t xs, int64_t M, int K, float* W,
                                float* b, int N, bool relu, const float* Y, int64_t ys,
                                const void* dY, bool dy_bf16, int64_t dys, bool bf16, float lr,
                                float* dX, int64_t dxs, void* workspace, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int64_t chunks = (M + kColRows - 1) / kColRows;
  char* ws = static_cast<char*>(workspace);
  float* dA = reinterpret_cast<float*>(ws);
  float* colpart = reinterpret_cast<float*>(ws + round256((size_t)M * N * sizeof(float)));
  float* part = reinterpret_cast<float*>(ws + round256((size_t)M * N * sizeof(float)) +
                                         round256((size_t)chunks * N * sizeof(float)));
  // 1. dA and the bias gradient's column partials
  {
    const unsigned grid = (unsigned)(((N + 255) / 256) * chunks);
    if (dy_bf16)
      relu_bwd_kernel<true><<<grid, 256, 0, s>>>(dY, dys, Y, ys, M, N, relu, dA, colpart);
    else
      relu_bwd_kernel<false><<<grid, 256, 0, s>>>(dY, dys, Y, ys, M, N, relu, dA, colpart);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // 2. dX = dA W, with the weights before this step's update
  if (dX) {
    GemmArgs g{};
    g.A = dA;
    g.lda = N;
    g.B = W;
    g.ldb = K;
    g.M = M;
    g.N = K;
    g.K = N;
    g.C = dX;
    g.ldc = dxs;
    g.k_split = ((int64_t)N + kBK - 1) / kBK * kBK;
    g.vec_a = vec_ok(dA, N);
    g.vec_b = vec_ok(W, K);
    hipError_t e = launch_gemm<true, false, kStore>(bf16, g, 1, s);
    if (e != hipSuccess) return e;
  }
  // 3. W -= lr dA^T X: rows n of the layer's output, columns k of its input, reduced over m
  {
    int64_t ks = 0;
    const int S = dense_wgrad_splits(M, N, K, &ks);
    GemmArgs g{};
    g.A = dA;
    g.lda = N;
    g.B = X;
    g.ldb = xs;
    g.M = N;
    g.N = K;
    g.K = M;
    g.k_split = ks;
    g.lr = lr;
    g.vec_a = vec_ok(dA, N);
    g.vec_b = vec_ok(X, xs);
    hipError_t e;
    if (S == 1) {
      g.C = W;
      g.ldc = K;
      e = launch_gemm<false, false, kSgd>(bf16, g, 1, s);
    } else {
      g.C = part;
      g.ldc = K;
      e = launch_gemm<false, false, kPartial>(bf16, g, S, s);
      if (e == hipSuccess) {
        const int64_t count = (int64_t)N * K;
        sgd_from_partials_kernel<<<(unsigned)((count + 255) / 256), 256, 0, s>>>(part, count, S,
                                                                                 lr, W);
        e = hipGetLastError();
      }
    }
    if (e != hipSuccess) return e;
  }
  // 4. b -= lr sum_m dA
  if (b) {
    bias_sgd_kernel<<<(unsigned)((N + 255) / 256), 256, 0, s>>>(colpart, chunks, N, lr, b);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_logistic_ne(const float* logits, int64_t ls, const float* labels, int64_t M,
                              float* prob, float* dlogits, int64_t dls, float* stats,
                              hipStream_t s) {
  logistic_ne_kernel<<<1, kHeadThreads, 0, s>>>(logits, ls, labels, M, prob, dlogits, dls,
                                                stats);
  return hipGetLastError();
}

}  // namespace ctr
