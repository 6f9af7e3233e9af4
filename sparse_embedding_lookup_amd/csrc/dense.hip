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
// gradient carries the 1/M of the mean cross-entropy.  The backward is one elementwise
// pass and two GEMMs: dA (ReLU layers only) is written once in the GEMMs' operand type (bf16
// nearest-even for bf16 compute, the rounding the GEMMs apply anyway, so half the bytes),
// and the bias is the weight of a constant input 1, so its gradient is one more output
// column of the weight-gradient GEMM (the input X read with a column of ones appended).
//
// GEMMs run on the matrix cores.  A 256-thread block owns a 128x128 output tile: four
// waves of 64x64, each 2x2 MFMA tiles of 32x32.  The reduction advances in k-tiles of 32
// staged through two LDS buffers (one barrier per k-tile), with the next k-tile's global
// loads in flight during the current one's MFMAs.  fp32 compute: v_mfma_f32_32x32x2f32 on fp32 operands; bf16 compute:
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

constexpr int kBM = 128, kBN = 128;
// k-tile: 32.  A 64-wide bf16 k-tile doubles the bytes in flight per barrier, but its LDS
// (2 x 2 x 128 x 72 bf16) and registers leave two blocks per CU instead of three: the
// forward on a 32768 x 2208 x 1024 layer went from 0.364 to 0.433 ms.  With a transposed
// operand (KT/2 loads per thread) it would run one wave per SIMD.
__host__ __device__ constexpr int k_tile(bool, bool, bool) { return 32; }
constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;              // accelerator complex dies of the MI355X
constexpr int kHeadThreads = 1024;

// kSgd: C -= lr * acc (W, and the bias column), or, in a split reduction (gridDim.z > 1),
// the slice's partial sums at C[(z * M + m) * ldc + n].
enum Epilogue { kStore = 0, kBiasAct = 1, kSgd = 2 };

// C[m, n] (m < M, n < N) from A[m, k] and B[k, n] (k < K):
//   A[m, k] = AK ? A[m * lda + k] : A[k * lda + m]
//   B[k, n] = BK ? B[n * ldb + k] : B[k * ldb + n]
//   C[m, n] at C[m * ldc + n]
// A is fp32 (ASRC = kPlain) or bf16 (kPlainBF16, widened exactly as it is loaded).  B may
// have a row of ones: B[k, n] = 1 for n == ones_col (the bias column of the weight
// gradient).
enum Source { kPlain = 0, kPlainBF16 = 1 };

struct GemmArgs {
  const void* A;       // fp32 or bf16 (ASRC)
  int64_t lda;
  const float* B;
  int64_t ldb;
  int64_t M, N, K;
  float* C;
  int64_t ldc;
  const float* bias;   // kBiasAct, nullable
  int relu;            // kBiasAct
  float lr;            // kSgd
  int64_t k_split;     // reduction length per grid.z slice, a multiple of the k-tile
  int64_t n_tiles;     // output tiles along n (the block index runs along n first)
  int vec_a, vec_b;    // operand 16-byte aligned with a stride that is a multiple of 4
  int64_t ones_col;    // B: the column n that reads 1 (-1: none)
  int64_t wcols;       // kSgd: C columns n < wcols are W[m, n]; n == wcols is the bias b[m]
  float* bias_out;     //   (a split reduction writes both to the partial rows)
};

// Operand P[r, k] (r < rows, k < kend): KMAJ ? P[r * ld + k] : P[k * ld + r], fp32 or bf16
// (SRC).  Each thread loads KT/2 elements of the 128 x KT tile at (r0, k0) so that every
// load instruction reads consecutive addresses across the wavefront:
//   KMAJ: KT/8 runs of 4 consecutive k; KT/4 lanes share a row (one 16-byte or 8-byte load
//         per run when the operand allows it);
//   else: row t & 127 and the KT/2 consecutive k from (KT/2)(t >> 7), one load each (the
//         lanes of a wavefront read 64 consecutive rows).
// Elements outside the operand are zero, except that row `ones` reads 1.
struct Src {
  const void* p;
  int64_t ld, rows, ones;
  int vec;
};

template <int SRC>
__device__ __forceinline__ float fetch1(const Src& o, int64_t off) {
  if constexpr (SRC == kPlainBF16)
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(o.p)[off] << 16);
  else
    return static_cast<const float*>(o.p)[off];
}

template <int SRC>
__device__ __forceinline__ void fetch4(const Src& o, int64_t off, float* v) {
  if constexpr (SRC == kPlainBF16) {
    const uint2 h = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(o.p) + off);
    v[0] = bf16_lo(h.x); v[1] = bf16_hi(h.x); v[2] = bf16_lo(h.y); v[3] = bf16_hi(h.y);
  } else {
    const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(o.p) + off);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
}

template <bool KMAJ, int SRC, int KT, int ROWS>
__device__ __forceinline__ void load_tile(const Src& o, int64_t kend, int64_t r0, int64_t k0,
                                          float (&v)[ROWS * KT / kGemmThreads]) {
  constexpr int LPR = KT / 4;                       // KMAJ: lanes per row, 4 consecutive k
  constexpr int GROUPS = kGemmThreads / ROWS;       // else: threads per row
  constexpr int RUN = KT / GROUPS;                  //   and consecutive k per thread
  const int t = threadIdx.x;
  if constexpr (KMAJ) {
#pragma unroll
    for (int q = 0; q < ROWS * LPR / kGemmThreads; ++q) {
      const int64_t r = r0 + t / LPR + (kGemmThreads / LPR) * q;
      const int64_t k = k0 + 4 * (t % LPR);
      if (o.vec && r < o.rows && k + 3 < kend) {
        fetch4<SRC>(o, r * o.ld + k, v + 4 * q);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[4 * q + e] = (r < o.rows && k + e < kend) ? fetch1<SRC>(o, r * o.ld + k + e) : 0.f;
      }
    }
  } else {
    const int64_t r = r0 + (t % ROWS);
    const int64_t k = k0 + RUN * (t / ROWS);
    const bool rv = r < o.rows;
    const float outside = r == o.ones ? 1.f : 0.f;
    int64_t off = k * o.ld + r;
    if (rv && k + RUN <= kend) {              // the whole run is inside the operand
#pragma unroll
      for (int j = 0; j < RUN; ++j) {
        v[j] = fetch1<SRC>(o, off);
        off += o.ld;
      }
    } else {
#pragma unroll
      for (int j = 0; j < RUN; ++j) {
        v[j] = (k + j < kend) ? (rv ? fetch1<SRC>(o, off) : outside) : 0.f;
        off += o.ld;
      }
    }
  }
}

// The tile in LDS as [ROWS][PITCH], k contiguous, in the compute type (the conversion to
// bf16 is the nearest-even rounding of the operand).  Rows are 16-byte aligned: the KMAJ
// runs go out as one 8-byte (bf16) or 16-byte (fp32) store, the KT/2-k runs as 16-byte
// stores.
template <typename LT>
__device__ __forceinline__ void put(LT* dst, const float* x, int n) {
  if constexpr (std::is_same<LT, float>::value) {
    for (int i = 0; i < n; i += 4)
      *reinterpret_cast<float4*>(dst + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
  } else {
    for (int i = 0; i < n; i += 4) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 h = {(__bf16)x[i], (__bf16)x[i + 1], (__bf16)x[i + 2], (__bf16)x[i + 3]};
      *reinterpret_cast<bf16x4*>(dst + i) = h;
    }
  }
}

template <bool KMAJ, typename LT, int PITCH, int KT, int ROWS>
__device__ __forceinline__ void store_tile(LT* __restrict__ lds,
                                           const float (&v)[ROWS * KT / kGemmThreads]) {
  constexpr int LPR = KT / 4, RUN = KT / (kGemmThreads / ROWS);
  const int t = threadIdx.x;
  if constexpr (KMAJ) {
#pragma unroll
    for (int q = 0; q < ROWS * LPR / kGemmThreads; ++q)
      put<LT>(lds + (t / LPR + (kGemmThreads / LPR) * q) * PITCH + 4 * (t % LPR), v + 4 * q, 4);
  } else {
    put<LT>(lds + (t % ROWS) * PITCH + RUN * (t / ROWS), v, RUN);
  }
}

// TI: 32-row MFMA tiles per wave along m, so the block tile is (64 TI) x 128.  TI = 1 is for
// grids that 128-row tiles would leave with fewer blocks than compute units.
template <bool BF, bool AK, bool BK, int EPI, int ASRC, int TI>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmArgs g) {
  using LT = typename std::conditional<BF, __bf16, float>::type;
  constexpr int KT = k_tile(BF, AK, BK);
  constexpr int BMT = 64 * TI;
  // rows of 16-byte multiples, padded against bank conflicts of the fragment reads
  constexpr int PITCH = BF ? KT + 8 : KT + 4;
  constexpr int TILEA = BMT * PITCH, TILEB = kBN * PITCH;
  __shared__ __attribute__((aligned(16))) LT As[2 * TILEA];  // two buffers: one barrier
  __shared__ __attribute__((aligned(16))) LT Bs[2 * TILEB];  // per k-tile

  // Blocks go to the 8 XCDs round-robin (block b to XCD b mod 8), each with its own L2.
  // Give each XCD a contiguous run of tiles: the tiles that share an A row block (same m,
  // consecutive n) then meet in one L2 instead of fetching it once per XCD.
  const int64_t nb = (int64_t)gridDim.x, b = blockIdx.x, per = nb / kXcds;
  const int64_t tile = b < per * kXcds ? (b % kXcds) * per + b / kXcds : b;
  const int64_t n0 = (tile % g.n_tiles) * kBN;
  const int64_t m0 = (tile / g.n_tiles) * BMT;
  const int64_t kb = (int64_t)blockIdx.z * g.k_split;
  const int64_t ke = g.K < kb + g.k_split ? g.K : kb + g.k_split;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = wv >> 1, wn = wv & 1, rl = lane & 31, kg = lane >> 5;

  f32x16 acc[TI][2];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const Src sa{g.A, g.lda, g.M, -1, g.vec_a};
  const Src sb{g.B, g.ldb, g.ones_col >= 0 ? g.ones_col : g.N, g.ones_col, g.vec_b};
  float va[BMT * KT / kGemmThreads], vb[kBN * KT / kGemmThreads];
  int cur = 0;
  if (kb < ke) {
    load_tile<AK, ASRC, KT, BMT>(sa, ke, m0, kb, va);
    load_tile<BK, kPlain, KT, kBN>(sb, ke, n0, kb, vb);
    store_tile<AK, LT, PITCH, KT, BMT>(As, va);
    store_tile<BK, LT, PITCH, KT, kBN>(Bs, vb);
  }
  __syncthreads();
  for (int64_t k0 = kb; k0 < ke; k0 += KT) {
    const bool more = k0 + KT < ke;
    if (more) {                          // next k-tile's loads overlap this tile's MFMAs
      load_tile<AK, ASRC, KT, BMT>(sa, ke, m0, k0 + KT, va);
      load_tile<BK, kPlain, KT, kBN>(sb, ke, n0, k0 + KT, vb);
    }
    const LT* Ac = As + cur * TILEA;
    const LT* Bc = Bs + cur * TILEB;
    if constexpr (BF) {
      // fragment: lane holds row rl, k = 16 s + 8 kg .. +8 (A: rows m, B: rows n of Bs)
#pragma unroll
      for (int s = 0; s < KT / 16; ++s) {
        bf16x8 a[TI], b[2];
#pragma unroll
        for (int i = 0; i < TI; ++i)
          a[i] = *reinterpret_cast<const bf16x8*>(Ac + (32 * TI * wm + 32 * i + rl) * PITCH +
                                                  16 * s + 8 * kg);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          b[j] = *reinterpret_cast<const bf16x8*>(Bc + (64 * wn + 32 * j + rl) * PITCH +
                                                  16 * s + 8 * kg);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    } else {
      // fragment: lane holds row rl, k = 2 s + kg
#pragma unroll
      for (int s = 0; s < KT / 2; ++s) {
        float a[TI], b[2];
#pragma unroll
        for (int i = 0; i < TI; ++i) a[i] = Ac[(32 * TI * wm + 32 * i + rl) * PITCH + 2 * s + kg];
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = Bc[(64 * wn + 32 * j + rl) * PITCH + 2 * s + kg];
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    }
    if (more) {                          // the other buffer was last read before the
      store_tile<AK, LT, PITCH, KT, BMT>(As + (cur ^ 1) * TILEA, va);   // previous barrier
      store_tile<BK, LT, PITCH, KT, kBN>(Bs + (cur ^ 1) * TILEB, vb);
    }
    __syncthreads();
    cur ^= 1;
  }

  // acc[i][j][v] = C[m, n]: m = 8 (v / 4) + 4 kg + v % 4 and n = rl within the 32x32 tile
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + 64 * wn + 32 * j + rl;
      if (n >= g.N) continue;
      float bn = 0.f;
      if constexpr (EPI == kBiasAct) bn = g.bias ? g.bias[n] : 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + 32 * TI * wm + 32 * i + 8 * (v >> 2) + 4 * kg + (v & 3);
        if (m >= g.M) continue;
        float x = acc[i][j][v];
        if constexpr (EPI == kStore) {
          if (gridDim.z > 1)             // a slice of a split reduction: its partial sum
            g.C[((int64_t)blockIdx.z * g.M + m) * g.ldc + n] = x;
          else
            g.C[m * g.ldc + n] = x;
        } else if constexpr (EPI == kBiasAct) {
          x += bn;
          if (g.relu) x = x > 0.f ? x : 0.f;
          g.C[m * g.ldc + n] = x;
        } else {
          if (gridDim.z > 1) {           // a slice of a split reduction: its partial sum
            g.C[((int64_t)blockIdx.z * g.M + m) * g.ldc + n] = x;
          } else {
            float* c = n < g.wcols ? g.C + m * g.ldc + n : g.bias_out + m;
            *c = __builtin_fmaf(-g.lr, x, *c);
          }
        }
      }
    }
}

// The update from the split weight gradient: part[s] is [N, cols] (cols = K, plus the bias
// column K when b is given); element (n, c) is summed over the S slices in order and applied
// to W[n, c] (c < K) or b[n] (c == K).
__global__ __launch_bounds__(256) void sgd_from_partials_kernel(
    const float* __restrict__ part, int64_t N, int64_t K, int64_t cols, int S, float lr,
    float* __restrict__ W, float* __restrict__ b) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t count = N * cols;
  if (i >= count) return;
  float s = 0.f;
  for (int z = 0; z < S; ++z) s += part[z * count + i];
  const int64_t n = i / cols, c = i - n * cols;
  float* t = c < K ? W + n * K + c : b + n;
  *t = __builtin_fmaf(-lr, s, *t);
}

// dX from the split dX reduction: part[s] is [M, K]; dX[m * dxs + k] = the sum over the S
// slices, in order.
__global__ __launch_bounds__(256) void sum_slices_kernel(const float* __restrict__ part,
                                                         int64_t M, int64_t K, int S,
                                                         float* __restrict__ dX, int64_t dxs) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t count = M * K;
  if (i >= count) return;
  float s = 0.f;
  for (int z = 0; z < S; ++z) s += part[z * count + i];
  const int64_t m = i / K, k = i - m * K;
  dX[m * dxs + k] = s;
}

// dA[m, n] = dY[m, n] * [Y[m, n] > 0], contiguous [M, N], fp32 or bf16 nearest-even (OUTB).
template <bool DYB, bool OUTB>
__global__ __launch_bounds__(256) void relu_grad_kernel(const void* __restrict__ dY, int64_t dys,
                                                        const float* __restrict__ Y, int64_t ys,
                                                        int64_t M, int64_t N,
                                                        void* __restrict__ dA) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * N) return;
  const int64_t m = i / N, n = i - m * N;
  float gv;
  if constexpr (DYB)
    gv = __uint_as_float((uint32_t)static_cast<const uint16_t*>(dY)[m * dys + n] << 16);
  else
    gv = static_cast<const float*>(dY)[m * dys + n];
  const float yv = Y[m * ys + n];
  gv = yv > 0.f ? gv : 0.f;
  if constexpr (OUTB)
    static_cast<__bf16*>(dA)[i] = (__bf16)gv;
  else
    static_cast<float*>(dA)[i] = gv;
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
  // four elements per thread per round, all loads issued before any is used
  constexpr int U = 4;
  for (int64_t i0 = t; i0 < M; i0 += (int64_t)U * kHeadThreads) {
    float xs[U], ls[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + (int64_t)u * kHeadThreads;
      const int64_t ic = i < M ? i : M - 1;
      xs[u] = s[ic * ss];
      ls[u] = y[ic];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + (int64_t)u * kHeadThreads;
      if (i >= M) break;
      const float x = xs[u], l = ls[u];
      const float e = expf(-fabsf(x));
      const float p = x >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
      ce += (fmaxf(x, 0.f) - l * x) + log1pf(e);
      ys += l;
      if (prob) prob[i] = p;
      if (dl) dl[i * dls] = (p - l) / fm;
    }
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

bool vec_ok(const void* p, int64_t ld, int elem_bytes) {
  return ((uintptr_t)p & (4 * elem_bytes - 1)) == 0 && (ld & 3) == 0;
}

// 64-row tiles when 128-row ones would leave fewer blocks than compute units (forward and
// dX; the weight gradient fills the chip by splitting its reduction instead).
template <bool AK, bool BK, int EPI, int ASRC>
hipError_t launch_gemm(bool bf16, GemmArgs g, int splits, hipStream_t s) {
  g.n_tiles = (g.N + kBN - 1) / kBN;
  const int64_t tiles = g.n_tiles * ((g.M + kBM - 1) / kBM);
  if (tiles == 0) return hipSuccess;
  if constexpr (EPI != kSgd) {
    if (tiles * splits < 256) {
      const dim3 grid((unsigned)(g.n_tiles * ((g.M + 63) / 64)), 1, (unsigned)splits);
      if (bf16)
        gemm_kernel<true, AK, BK, EPI, ASRC, 1><<<grid, kGemmThreads, 0, s>>>(g);
      else
        gemm_kernel<false, AK, BK, EPI, ASRC, 1><<<grid, kGemmThreads, 0, s>>>(g);
      return hipGetLastError();
    }
  }
  const dim3 grid((unsigned)tiles, 1, (unsigned)splits);
  if (bf16)
    gemm_kernel<true, AK, BK, EPI, ASRC, 2><<<grid, kGemmThreads, 0, s>>>(g);
  else
    gemm_kernel<false, AK, BK, EPI, ASRC, 2><<<grid, kGemmThreads, 0, s>>>(g);
  return hipGetLastError();
}

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

// Slices of the weight-gradient reduction over the M batch rows: none while the output
// tiles (N rows by `cols` columns) alone give a block per compute unit, else enough for
// about two blocks per unit (six when slices would be 4096 rows or longer), each slice at
// least 128 rows long.  *k_split: rows per slice
// (a multiple of the compute type's k-tile).
int dense_wgrad_splits(int64_t M, int N, int cols, bool bf16, int64_t* k_split) {
  const int kt = k_tile(bf16, false, false);
  const int64_t tiles = (int64_t)((N + kBM - 1) / kBM) * ((cols + kBN - 1) / kBN);
  int64_t S = 1;
  if (tiles < 256) {
    const int64_t cap = M / 128 > 1 ? M / 128 : 1;
    S = (512 + tiles - 1) / tiles;
    if (S > cap) S = cap;
    // long slices: aim for about six blocks per unit instead, so that the last blocks of
    // the grid do not leave units idle for a whole long slice (a 32768 x 2208 -> 1024
    // layer's weight GEMM went from 0.97 to 0.72 ms; shorter slices gain nothing)
    if (M / S >= 4096) {
      S = (1536 + tiles - 1) / tiles;
      if (S > cap) S = cap;
    }
  }
  int64_t ks = (M + S - 1) / S;
  ks = (ks + kt - 1) / kt * kt;
  if (ks < kt) ks = kt;
  S = (M + ks - 1) / ks;
  if (S < 1) S = 1;
  if (k_split) *k_split = ks;
  return (int)S;
}

// Workspace of the backward: dA (ReLU layers: M * N in the compute type), then the split
// reduction's partials.
// Slices of dX's reduction over the layer's N outputs when its output tiles (M rows by K
// columns) alone are too few to fill the chip: about two blocks per unit, each slice at
// least 128 outputs long.  *k_split: outputs per slice (a multiple of the k-tile).
int dense_dx_splits(int64_t M, int N, int K, int64_t* k_split) {
  const int kt = k_tile(false, true, false);
  const int64_t tiles = ((M + kBM - 1) / kBM) * (int64_t)((K + kBN - 1) / kBN);
  int64_t S = 1;
  if (tiles > 0 && tiles < 256) {      // M = 0: no tiles, nothing to split
    const int64_t cap = N / 128 > 1 ? N / 128 : 1;
    S = (512 + tiles - 1) / tiles;
    if (S > cap) S = cap;
  }
  int64_t ks = (N + S - 1) / S;
  ks = (ks + kt - 1) / kt * kt;
  if (ks < kt) ks = kt;
  S = (N + ks - 1) / ks;
  if (S < 1) S = 1;
  if (k_split) *k_split = ks;
  return (int)S;
}

// The backward's workspace: dA (ReLU layers), then the weight gradient's partials, then dX's
// (both only when their reductions are split; dX's counted whether or not dX is asked for).
size_t dense_bwd_workspace_bytes(int64_t M, int N, int K, bool bias, bool relu, bool bf16) {
  const int cols = K + (bias ? 1 : 0);
  const int S = dense_wgrad_splits(M, N, cols, bf16, nullptr);
  const int Sx = dense_dx_splits(M, N, K, nullptr);
  const size_t da = relu ? round256((size_t)M * N * (bf16 ? 2 : 4)) : 0;
  const size_t part = S > 1 ? round256((size_t)S * N * cols * sizeof(float)) : 0;
  const size_t partx = Sx > 1 ? round256((size_t)Sx * M * K * sizeof(float)) : 0;
  return da + part + partx > 0 ? da + part + partx : 256;
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
  const int kt = k_tile(bf16, true, true);
  g.k_split = ((int64_t)K + kt - 1) / kt * kt;
  g.vec_a = vec_ok(X, xs, 4);
  g.vec_b = vec_ok(W, K, 4);
  g.ones_col = -1;
  return launch_gemm<true, true, kBiasAct, kPlain>(bf16, g, 1, s);
}

hipError_t launch_dense_bwd_sgd(const float* X, int64_t xs, int64_t M, int K, float* W,
                                float* b, int N, bool relu, const float* Y, int64_t ys,
                                const void* dY, bool dy_bf16, int64_t dys, bool bf16, float lr,
                                float* dX, int64_t dxs, void* workspace, hipStream_t s) {
  if (M == 0) return hipSuccess;
  char* ws = static_cast<char*>(workspace);
  // 1. the GEMMs' dA operand: dY itself for a linear layer, else dY * [Y > 0] written once
  const void* dA = dY;
  int64_t lda = dys;
  bool a_bf16 = dy_bf16;
  size_t used = 0;
  if (relu) {
    const int64_t count = M * (int64_t)N;
    const unsigned blocks = (unsigned)((count + 255) / 256);
    if (dy_bf16 && bf16)
      relu_grad_kernel<true, true><<<blocks, 256, 0, s>>>(dY, dys, Y, ys, M, N, ws);
    else if (dy_bf16)
      relu_grad_kernel<true, false><<<blocks, 256, 0, s>>>(dY, dys, Y, ys, M, N, ws);
    else if (bf16)
      relu_grad_kernel<false, true><<<blocks, 256, 0, s>>>(dY, dys, Y, ys, M, N, ws);
    else
      relu_grad_kernel<false, false><<<blocks, 256, 0, s>>>(dY, dys, Y, ys, M, N, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dA = ws;
    lda = N;
    a_bf16 = bf16;
    used = round256((size_t)count * (bf16 ? 2 : 4));
  }
  auto gemm = [&](auto AK, auto BK, auto EPI, GemmArgs g, int splits) {
    constexpr bool ak = decltype(AK)::value, bk = decltype(BK)::value;
    constexpr int epi = decltype(EPI)::value;
    return a_bf16 ? launch_gemm<ak, bk, epi, kPlainBF16>(bf16, g, splits, s)
                  : launch_gemm<ak, bk, epi, kPlain>(bf16, g, splits, s);
  };
  using T = std::true_type;
  using F = std::false_type;
  using Store = std::integral_constant<int, kStore>;
  using Sgd = std::integral_constant<int, kSgd>;
  // the weight gradient's split (its partials follow dA in the workspace, dX's follow those)
  const int cols = K + (b ? 1 : 0);
  int64_t ks = 0;
  const int S = dense_wgrad_splits(M, N, cols, bf16, &ks);
  const size_t wpart = S > 1 ? round256((size_t)S * N * cols * sizeof(float)) : 0;
  // 2. dX = dA W, with the weights before this step's update (A = dA rows, k = n)
  if (dX) {
    GemmArgs g{};
    g.A = dA;
    g.lda = lda;
    g.B = W;
    g.ldb = K;
    g.M = M;
    g.N = K;
    g.K = N;
    int64_t ksx = 0;
    const int Sx = dense_dx_splits(M, N, K, &ksx);
    float* partx = reinterpret_cast<float*>(ws + used + wpart);
    g.C = Sx > 1 ? partx : dX;
    g.ldc = Sx > 1 ? K : dxs;
    g.k_split = ksx;
    g.vec_a = vec_ok(dA, lda, a_bf16 ? 2 : 4);
    g.vec_b = vec_ok(W, K, 4);
    g.ones_col = -1;
    hipError_t e = gemm(T{}, F{}, Store{}, g, Sx);
    if (e != hipSuccess) return e;
    if (Sx > 1) {
      const int64_t count = M * (int64_t)K;
      sum_slices_kernel<<<(unsigned)((count + 255) / 256), 256, 0, s>>>(partx, M, K, Sx, dX,
                                                                        dxs);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  // 3. [W | b] -= lr dA^T [X | 1]: rows n of the layer's output, columns k of its input and
  //    the bias column K, reduced over the m rows (A[n, m] = dA[m, n], B[m, k] = X[m, k])
  GemmArgs g{};
  g.A = dA;
  g.lda = lda;
  g.B = X;
  g.ldb = xs;
  g.M = N;
  g.N = cols;
  g.K = M;
  g.k_split = ks;
  g.lr = lr;
  g.vec_a = 0;                         // the transposed operands load one element per lane
  g.vec_b = 0;
  g.ones_col = b ? K : -1;
  g.wcols = K;
  g.bias_out = b;
  if (S == 1) {
    g.C = W;
    g.ldc = K;
    return gemm(F{}, F{}, Sgd{}, g, 1);
  }
  float* part = reinterpret_cast<float*>(ws + used);
  g.C = part;
  g.ldc = cols;
  hipError_t e = gemm(F{}, F{}, Sgd{}, g, S);
  if (e != hipSuccess) return e;
  const int64_t count = (int64_t)N * cols;
  sgd_from_partials_kernel<<<(unsigned)((count + 255) / 256), 256, 0, s>>>(part, N, K, cols, S,
                                                                           lr, W, b);
  return hipGetLastError();
}

hipError_t launch_logistic_ne(const float* logits, int64_t ls, const float* labels, int64_t M,
                              float* prob, float* dlogits, int64_t dls, float* stats,
                              hipStream_t s) {
  logistic_ne_kernel<<<1, kHeadThreads, 0, s>>>(logits, ls, labels, M, prob, dlogits, dls,
                                                stats);
  return hipGetLastError();
}

}  // namespace ctr
