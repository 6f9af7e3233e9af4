// fused.hip -- sum pooling and the pairwise-dot interaction in one pass on gfx950.
//
// Method: the pooled vectors of "DHEN" notes, 2.1 (one d-dim vector per sparse feature, sum
// pooling) feed the dot interaction of "Meta DLRM" (upskillscore.com), 02 and "DHEN" notes,
// 3.1 and Solution 2: R[b] = [ z_0 | <z_i, z_j> for F > i > j >= 0 ], z_0 the dense vector.
// Both steps compute what the separate calls compute; only the home of the pooled vectors
// between them changes.  The separate path writes Z and reads it back; here a block pools its
// samples' bags, writes them to Z (the backward reads Z) and keeps a copy in LDS that the
// dots are taken from, so the forward's second pass over Z disappears.
//
// Phase 1 (pooling).  A block owns S consecutive samples, so S*T bags, taken sample-major
// (bag c = s*T + t is global bag t*batch + b0 + s).  Their occurrences, concatenated in that
// order, are split evenly over the block's lane groups: G lanes per group, one 16-byte vector
// of the row per lane, kU row loads in flight.  A group adds the rows of its share in
// occurrence order; a bag that crosses a share edge is finished by the group holding its
// first piece (kept in registers), which adds the following groups' pieces from LDS in order.  A finished bag goes to
// Z (fp32) and to the LDS copy: rounded to bf16 (nearest-even) for the matrix-core dots, or
// fp32 for the fp32 dots.  The dense rows Z[b, 0, :] are read into the copy and passed
// through to R.
// Phase 2 (interaction).  bf16: one wavefront per 32x32 lower-triangle tile of one sample on
// v_mfma_f32_32x32x16_bf16, operands read from the LDS copy, fp32 accumulation, only i > j
// written.  fp32: four lanes per pair, each a chain of fused multiply-adds over every fourth
// column, then summed across the four.
#include "ctr_internal.h"

namespace ctr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kMaxBags = kThreads;          // bags per block: one per thread in the scan
constexpr int kBlockLds = 32768;            // block total aimed at: five blocks per CU
constexpr int kPoolLdsMax = 47104;          // with the static arrays (<= 16.1 KiB), under 64 KiB
constexpr double kRowsPerGroup = 128.0;     // occurrences per lane group aimed at
constexpr int64_t kMinBlocks = 2048;        // keep several blocks per CU where the batch allows
constexpr double kMinRowsPerGroup = 20.0;   // ... unless a group's share would be shorter

// Row i of the strict lower triangle that holds pair index q (i(i-1)/2 <= q < i(i+1)/2).
__device__ __forceinline__ int pair_row(int q) {
  int i = (int)((1.0f + sqrtf(1.0f + 8.0f * (float)q)) * 0.5f);
  while (i * (i - 1) / 2 > q) --i;
  while ((i + 1) * i / 2 <= q) ++i;
  return i;
}

template <bool TBF16>
__device__ __forceinline__ void add_vector(float* acc, const uint4& x) {
  if (TBF16) {
    acc[0] += bf16_lo(x.x); acc[1] += bf16_hi(x.x);
    acc[2] += bf16_lo(x.y); acc[3] += bf16_hi(x.y);
    acc[4] += bf16_lo(x.z); acc[5] += bf16_hi(x.z);
    acc[6] += bf16_lo(x.w); acc[7] += bf16_hi(x.w);
  } else {
    acc[0] += __uint_as_float(x.x); acc[1] += __uint_as_float(x.y);
    acc[2] += __uint_as_float(x.z); acc[3] += __uint_as_float(x.w);
  }
}

// TBF16: table stored as bf16.  G: lanes per row (dim = G * values per vector).  FB > 0:
// matrix-core dots over FB 32-row blocks and KS k-steps of 16 (dim = 16 * KS); FB == 0:
// fp32 dots.  Z is [batch, F, dim] fp32 with F = T + 1.
// Rows of 16 or more vectors: the kernel fits 96 registers without spilling, so five waves
// per SIMD keep more row loads in flight; narrower rows (16 loads in flight per group) keep
// the registers they need.
template <bool TBF16, int G, int FB, int KS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(G >= 16 ? 5 : 1)))
void embbag_interaction_fwd_kernel(
    const char* __restrict__ table, int64_t total_rows, const int64_t* __restrict__ row_base,
    int T, const void* __restrict__ idxv, bool idx64, int64_t nnz,
    const int64_t* __restrict__ offsets, int64_t batch, int S, float* __restrict__ Z,
    float* __restrict__ R, int64_t r_stride) {
  constexpr int E = TBF16 ? 8 : 4;           // table values per 16-byte vector
  constexpr int dim = G * E;
  constexpr int kGroups = kThreads / G;
  constexpr int kU = G <= 8 ? 16 : 8;        // rows in flight per group
  constexpr int kRegs = (kU + G - 1) / G;
  constexpr bool kMfma = FB > 0;
  constexpr int kPitchH = dim + 8;           // bf16 copy: row pitch in bf16 (16-byte pad)
  constexpr int kPitchF = dim + 1;           // fp32 copy: row pitch in floats (1-float pad)
  static_assert(!kMfma || dim == 16 * KS, "matrix-core shape");
  extern __shared__ __align__(16) unsigned char s_pool[];
  __shared__ int32_t s_beg[kMaxBags];
  __shared__ int64_t s_vpre[kMaxBags + 1];   // bag c: [s_vpre[c], s_vpre[c+1]) of the concatenation
  __shared__ int64_t s_base[kMaxBags];
  __shared__ float s_first[kGroups][dim];    // piece that began before the share
  __shared__ int32_t s_fbag[kGroups], s_fcont[kGroups];
  __shared__ int64_t s_wsum[kThreads / 64];

  const int F = T + 1;
  const int tid = threadIdx.x;
  const int lane = tid & (G - 1), grp = tid / G;
  const int lane0 = (tid & 63) & ~(G - 1);
  const int64_t b0 = (int64_t)blockIdx.x * S;
  const int ns = (int)clamp64(batch - b0, 0, S);
  const int nb = ns * T;                     // <= kMaxBags (host)
  __bf16* poolh = reinterpret_cast<__bf16*>(s_pool);
  float* poolf = reinterpret_cast<float*>(s_pool);

  // bag table: first occurrence, row base, and an exclusive scan of the lengths
  int64_t len = 0;
  if (tid < nb) {
    const int s = tid / T, t = tid - s * T;
    const int64_t g = (int64_t)t * batch + b0 + s;
    const int64_t o0 = clamp64(offsets[g], 0, nnz), o1 = clamp64(offsets[g + 1], 0, nnz);
    s_beg[tid] = (int32_t)o0;
    s_base[tid] = row_base ? row_base[t] : 0;
    len = o1 > o0 ? o1 - o0 : 0;
  }
  int64_t x = len;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t y = __shfl_up(x, d, 64);
    if ((tid & 63) >= d) x += y;
  }
  if ((tid & 63) == 63) s_wsum[tid >> 6] = x;
  // dense rows: the copy's row 0 and R[b, 0:dim] (exact)
  for (int e = tid; e < ns * dim; e += kThreads) {
    const int s = e / dim, c = e - s * dim;
    const int64_t b = b0 + s;
    const float v = Z[b * F * dim + c];
    R[b * r_stride + c] = v;
    if (kMfma) poolh[(s * F) * kPitchH + c] = (__bf16)v;
    else poolf[(s * F) * kPitchF + c] = v;
  }
  __syncthreads();
  {
    int64_t add = 0;
    for (int w = 0; w < (tid >> 6); ++w) add += s_wsum[w];
    if (tid < nb) s_vpre[tid + 1] = x + add;
    if (tid == 0) s_vpre[0] = 0;
  }
  __syncthreads();

  // a finished bag: Z row (fp32, 16-byte stores) and the LDS copy
  auto emit = [&](int c, const float (&acc)[E]) {
    const int s = c / T, t = c - s * T;
    const int row = s * F + 1 + t;
    float* o = Z + (b0 * F + row) * dim + lane * E;
    reinterpret_cast<float4*>(o)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    if (E == 8)
      reinterpret_cast<float4*>(o)[1] = make_float4(acc[4 % E], acc[5 % E], acc[6 % E], acc[7 % E]);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (kMfma) poolh[row * kPitchH + lane * E + e] = (__bf16)acc[e];
      else poolf[row * kPitchF + lane * E + e] = acc[e];
    }
  };
  auto to_lds = [&](float* dst, const float (&acc)[E]) {
#pragma unroll
    for (int e = 0; e < E; ++e) dst[lane * E + e] = acc[e];
  };
  auto index_at = [&](int64_t k) -> int64_t {
    return idx64 ? static_cast<const int64_t*>(idxv)[k]
                 : (int64_t) static_cast<const int32_t*>(idxv)[k];
  };

  const int64_t L = s_vpre[nb];
  const int64_t share = (L + kGroups - 1) / kGroups;
  const int64_t q0 = (int64_t)grp * share;
  const int64_t q1 = q0 + share < L ? q0 + share : L;
  int32_t fbag = -1, fcont = 0, lbag = -1;
  float lacc[E];                             // piece that continues past the share
#pragma unroll
  for (int e = 0; e < E; ++e) lacc[e] = 0.f;
  if (q0 < q1) {
    // bag of the share's first position: last c with s_vpre[c] <= q0
    int c = 0, hi = nb - 1;
    while (c < hi) {
      const int mid = (c + hi + 1) >> 1;
      if (s_vpre[mid] <= q0) c = mid; else hi = mid - 1;
    }
    bool piece_at_start = q0 == s_vpre[c];
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    auto close_piece = [&](bool bag_ends_here) {
      if (piece_at_start && bag_ends_here) {
        emit(c, acc);
      } else if (!piece_at_start) {            // began before this share
        fbag = c;
        fcont = bag_ends_here ? 0 : 1;
        to_lds(s_first[grp], acc);
      } else {                                 // began here, continues past the share
        lbag = c;
#pragma unroll
        for (int e = 0; e < E; ++e) lacc[e] = acc[e];
      }
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = 0.f;
    };
    for (int64_t k0 = q0; k0 < q1; k0 += kU) {
      // indices of the window, loaded cooperatively and broadcast by shuffles
      int64_t iv[kRegs];
#pragma unroll
      for (int r = 0; r < kRegs; ++r) {
        const int e = r * G + lane;
        const int64_t v = k0 + e;
        iv[r] = 0;
        if (e < kU && v < q1) {
          int ce = c;
          while (ce < nb - 1 && v >= s_vpre[ce + 1]) ++ce;
          iv[r] = index_at(s_beg[ce] + (v - s_vpre[ce]));
        }
      }
      uint4 rv[kU];
      int bagu[kU];
      int cc = c;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t v = k0 + u;
        while (cc < nb - 1 && v >= s_vpre[cc + 1]) ++cc;
        bagu[u] = cc;
        const int64_t id = __shfl(iv[u / G], lane0 + (u % G), 64);
        const int64_t key = s_base[cc] + id;
        const bool live = v < q1;
        const bool ok = key >= 0 && key < total_rows;
        if (live && ok)
          rv[u] = *reinterpret_cast<const uint4*>(table + key * (int64_t)(dim * (TBF16 ? 2 : 4)) +
                                                  (int64_t)lane * 16);
        else if (live)
          rv[u] = make_uint4(0x7FC00000u, 0x7FC00000u, 0x7FC00000u, 0x7FC00000u);  // NaN
        else
          rv[u] = make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (k0 + u >= q1) break;
        if (bagu[u] != c) {                    // the piece of bag c ended at this position
          close_piece(true);
          c = bagu[u];
          piece_at_start = true;
        }
        add_vector<TBF16>(acc, rv[u]);
      }
    }
    close_piece(q1 == s_vpre[c + 1]);
  }
  if (lane == 0) {
    s_fbag[grp] = fbag;
    s_fcont[grp] = fcont;
  }
  __syncthreads();
  if (lbag != -1) {
    for (int j = grp + 1; j < kGroups && s_fbag[j] == lbag; ++j) {
#pragma unroll
      for (int e = 0; e < E; ++e) lacc[e] += s_first[j][lane * E + e];
      if (!s_fcont[j]) break;
    }
    emit(lbag, lacc);
  }
  // empty bags: zeros
  for (int j = tid; j < nb; j += kThreads) {
    if (s_vpre[j] == s_vpre[j + 1]) {
      const int s = j / T, t = j - s * T;
      const int row = s * F + 1 + t;
      float* o = Z + (b0 * F + row) * dim;
      for (int c2 = 0; c2 < dim; c2 += 4)
        *reinterpret_cast<float4*>(o + c2) = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int c2 = 0; c2 < dim; ++c2) {
        if (kMfma) poolh[row * kPitchH + c2] = (__bf16)0.f;
        else poolf[row * kPitchF + c2] = 0.f;
      }
    }
  }
  __syncthreads();

  if constexpr (kMfma) {
    constexpr int kTiles = FB * (FB + 1) / 2;
    const int wave = tid >> 6, ln = tid & 63, rl = ln & 31, kg = ln >> 5;
    for (int q = wave; q < ns * kTiles; q += kThreads / 64) {
      const int s = q / kTiles;
      int J = q - s * kTiles, I = 0;
      while (J > I) { J -= I + 1; ++I; }       // tile (I, J), J <= I
      if (J == I && F - 32 * I < 2) continue;  // no pair i > j inside this tile
      bf16x8 fa[KS], fb[KS];
      const int ra = 32 * I + rl, rb = 32 * J + rl;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const int col = 16 * k + 8 * kg;
        bf16x8 z = {};
        fa[k] = ra < F ? *reinterpret_cast<const bf16x8*>(poolh + (s * F + ra) * kPitchH + col) : z;
        fb[k] = rb < F ? *reinterpret_cast<const bf16x8*>(poolh + (s * F + rb) * kPitchH + col) : z;
      }
      f32x16 acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
      for (int k = 0; k < KS; ++k)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[k], fb[k], acc, 0, 0, 0);
      // acc[v] = D[m][n]: m = 8*(v/4) + 4*kg + v%4 (row of block I), n = rl (row of block J)
      float* rbp = R + (b0 + s) * r_stride + dim;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = 32 * I + 8 * (v >> 2) + 4 * kg + (v & 3);
        if (i < F && rb < i) rbp[i * (i - 1) / 2 + rb] = acc[v];
      }
    }
  } else {
    // four lanes per dot (columns k = part mod 4, fused multiply-adds in column order),
    // joined by two shuffles; a quad of lanes is always active together
    const int P = F * (F - 1) / 2;
    for (int e4 = tid; e4 < ns * P * 4; e4 += kThreads) {
      const int e = e4 >> 2, part = e4 & 3;
      const int s = e / P, q = e - s * P;
      const int i = pair_row(q), j = q - i * (i - 1) / 2;
      const float* zi = poolf + (s * F + i) * kPitchF;
      const float* zj = poolf + (s * F + j) * kPitchF;
      float a = 0.f;
#pragma unroll 4
      for (int k = part; k < dim; k += 4) a = fmaf(zi[k], zj[k], a);
      a += __shfl_xor(a, 1, 64);
      a += __shfl_xor(a, 2, 64);
      if (part == 0) R[(b0 + s) * r_stride + dim + q] = a;
    }
  }
}

struct FusedShape {
  bool ok;
  int G;
  int S;
  size_t lds;
};

FusedShape fused_shape(int T, int dim, bool tbf16, bool bf16, int64_t batch, int64_t nnz) {
  FusedShape f{false, 0, 1, 0};
  const int E = tbf16 ? 8 : 4;
  const int F = T + 1;
  if (T < 1 || T > kMaxBags || dim % E) return f;
  const int G = dim / E;
  if (G < 1 || G > 32 || (G & (G - 1))) return f;
  if (bf16 && !(dim == 16 || dim == 32 || dim == 64 || dim == 128)) return f;
  if (bf16 && F > 128) return f;
  const size_t per = bf16 ? (size_t)F * (dim + 8) * 2 : (size_t)F * (dim + 1) * 4;
  if (per > (size_t)kPoolLdsMax) return f;
  const int kGroups = kThreads / G;
  // static arrays: the piece buffer (256 * E floats) and the bag table (about 5.2 KiB)
  const size_t fixed = (size_t)kThreads * E * 4 + 5376;
  int S = (int)((kBlockLds - (int)fixed) / (int)per);
  if (S < 1) S = 1;
  const double rows = batch > 0 ? (double)nnz / (double)batch : 1.0;
  const int s_rows = (int)(kRowsPerGroup * kGroups / (rows > 1.0 ? rows : 1.0)) + 1;
  if (s_rows < S) S = s_rows;
  const int64_t s_blocks = batch / kMinBlocks;
  if (s_blocks < S) S = (int)(s_blocks > 1 ? s_blocks : 1);
  // a share shorter than kMinRowsPerGroup leaves the load window half empty: take more
  // samples per block (fewer blocks) then, within the LDS budget
  const int s_lds = (int)(((size_t)kBlockLds - fixed) / per) > 1
                        ? (int)(((size_t)kBlockLds - fixed) / per) : 1;
  int s_min = (int)(kMinRowsPerGroup * kGroups / (rows > 1.0 ? rows : 1.0) + 0.999);
  if (s_min > s_lds) s_min = s_lds;
  if (S < s_min) S = s_min;
  if (S > kMaxBags / T) S = kMaxBags / T;
  if (S < 1) S = 1;
  f.ok = true;
  f.G = G;
  f.S = S;
  f.lds = per * S;
  return f;
}

template <bool TB, int G, int FB, int KS>
void launch_one(unsigned blocks, size_t lds, hipStream_t s, const char* table, int64_t total_rows,
                const int64_t* row_base, int T, const void* idx, bool idx64, int64_t nnz,
                const int64_t* offsets, int64_t batch, int S, float* Z, float* R,
                int64_t r_stride) {
  embbag_interaction_fwd_kernel<TB, G, FB, KS><<<blocks, kThreads, lds, s>>>(
      table, total_rows, row_base, T, idx, idx64, nnz, offsets, batch, S, Z, R, r_stride);
}

}  // namespace

bool embbag_interaction_supported(int num_tables, int dim, bool table_bf16, bool bf16) {
  return fused_shape(num_tables, dim, table_bf16, bf16, 1, 1).ok;
}

hipError_t launch_embbag_interaction_fwd(const void* table, bool table_bf16, int64_t total_rows,
                                         int dim, const int64_t* row_base, int num_tables,
                                         const void* idx, bool idx64, int64_t nnz,
                                         const int64_t* offsets, int64_t batch, float* Z,
                                         bool bf16, float* R, int64_t r_stride, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  const FusedShape f = fused_shape(num_tables, dim, table_bf16, bf16, batch, nnz);
  if (!f.ok) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)((batch + f.S - 1) / f.S);
  const char* tb = static_cast<const char*>(table);
  const int F = num_tables + 1;
#define CTR_FUSED_ARGS blocks, f.lds, s, tb, total_rows, row_base, num_tables, idx, idx64, nnz, \
                       offsets, batch, f.S, Z, R, r_stride
  if (bf16) {
    const int FB = (F + 31) / 32, KS = dim / 16;
#define CTR_FUSED_KS(TB_, FB_)                                                     \
  switch (KS) {                                                                    \
    case 1: launch_one<TB_, TB_ ? 2 : 4, FB_, 1>(CTR_FUSED_ARGS); break;           \
    case 2: launch_one<TB_, TB_ ? 4 : 8, FB_, 2>(CTR_FUSED_ARGS); break;           \
    case 4: launch_one<TB_, TB_ ? 8 : 16, FB_, 4>(CTR_FUSED_ARGS); break;          \
    default: launch_one<TB_, TB_ ? 16 : 32, FB_, 8>(CTR_FUSED_ARGS); break;        \
  }
#define CTR_FUSED_FB(TB_)                            \
  switch (FB) {                                      \
    case 1: CTR_FUSED_KS(TB_, 1) break;              \
    case 2: CTR_FUSED_KS(TB_, 2) break;              \
    case 3: CTR_FUSED_KS(TB_, 3) break;              \
    default: CTR_FUSED_KS(TB_, 4) break;             \
  }
    if (table_bf16) { CTR_FUSED_FB(true) } else { CTR_FUSED_FB(false) }
#undef CTR_FUSED_FB
#undef CTR_FUSED_KS
  } else {
#define CTR_FUSED_G(TB_)                                        \
  switch (f.G) {                                                \
    case 1: launch_one<TB_, 1, 0, 0>(CTR_FUSED_ARGS); break;    \
    case 2: launch_one<TB_, 2, 0, 0>(CTR_FUSED_ARGS); break;    \
    case 4: launch_one<TB_, 4, 0, 0>(CTR_FUSED_ARGS); break;    \
    case 8: launch_one<TB_, 8, 0, 0>(CTR_FUSED_ARGS); break;    \
    case 16: launch_one<TB_, 16, 0, 0>(CTR_FUSED_ARGS); break;  \
    default: launch_one<TB_, 32, 0, 0>(CTR_FUSED_ARGS); break;  \
  }
    if (table_bf16) { CTR_FUSED_G(true) } else { CTR_FUSED_G(false) }
#undef CTR_FUSED_G
  }
#undef CTR_FUSED_ARGS
  return hipGetLastError();
}

}  // namespace ctr
