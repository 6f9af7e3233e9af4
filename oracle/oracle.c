/*
 * oracle.c -- plain, slow CPU reference of the sparse front end of a CTR ranking model.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table or helper with
 * the HIP library; both sides read the same seeded inputs and nothing else.
 *
 * Every floating-point result is accumulated in double precision (fp32 inputs widen
 * exactly; fp32 x fp32 products are exact in fp64).  Beside each floating output the oracle
 * also returns a magnitude M = sum of |terms| (propagated from input magnitudes when those
 * are given), so that a result y is checked as |y_gpu - y| <= rtol * M.  This is the
 * textbook forward-error form of a floating-point sum, |s_hat - s| <= gamma_(n-1) * sum|x_i|.
 *
 * Sources (web pages, cited by title and section):
 *   [DHEN]  "DHEN" notes (calwoo.github.io), section 2.1 "Feature Processing Layer":
 *           each categorical term has a trainable d-dim vector; the dense features become
 *           one d-dim vector; the slot vectors are concatenated into X0 = (x_1..x_m).
 *           Section 3.1 "AdvancedDLRM" and Solution 2: inner products of all embedding
 *           pairs, the vector (s_ij)_{i<j} of length C(m,2), concatenated with the dense
 *           features; the squared-norm identity for the sum of all pair dots.
 *   [TN]    "How TensorNet Supercharges Sparse Feature Training on TensorFlow", section
 *           "Core Optimizations": collect the batch's IDs, sort them, give each a contiguous
 *           index (the virtual sparse feature), fetch the rows into a batch-sized matrix;
 *           section "Synchronous Architecture": only features present in the batch move.
 *   [DLRM]  "Meta DLRM" (upskillscore.com), section 02: the interaction is the dot product
 *           between all pairs of embedding vectors and the processed dense features.
 *           Section 3.1 also names the pair set i <= j with self-dots; Solution 2 the FM
 *           sum of all pair dots by the squared-norm identity.
 *           [TN] "Inference Optimization": online inference reads a pre-exported sparse
 *           embedding dictionary keyed by raw ID.
 *           Section 6.4 "Common Optimizations": low-precision (FP16) embedding storage
 *           whose updates use stochastic rounding.
 * Readings where the pages are silent (sum pooling, strict i > j pair order, sum of
 * gradients over the batch, RNE storage rounding, the stochastic-rounding rule and its
 * random bits) follow the plain definitions below.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ threads */
void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------ rounding */
/* Round a double to the nearest bfloat16 value (8 significant bits, exponent range of
 * binary32), ties to even, returned as a double.  Written from the IEEE-754 definition:
 * x = m * 2^e with 0.5 <= |m| < 1, keep 8 bits of m with round-half-even (rint in the
 * default rounding mode), below the normal range the quantum stays 2^-133. */
double orc_round_bf16(double x) {
  if (x == 0.0 || isnan(x) || isinf(x)) return x;
  int e;
  frexp(x, &e);
  int q = e - 8;                 /* exponent of the last kept bit */
  if (q < -133) q = -133;        /* subnormal bf16 quantum */
  double r = ldexp(rint(ldexp(x, -q)), q);
  if (fabs(r) > 3.3895313892515355e38) r = copysign(INFINITY, x); /* beyond bf16 max */
  return r;
}

/* Round a double to the nearest IEEE binary16 value (11 significant bits, exponents down to
 * -14, subnormal quantum 2^-24, largest finite 65504), ties to even, returned as a double.
 * The same construction as orc_round_bf16: keep 11 bits of m in x = m * 2^e with rint, the
 * quantum no finer than 2^-24; a result beyond 65504 is infinity.  ("DHEN" notes, 6.4 names
 * FP16 embedding storage.) */
double orc_round_f16(double x) {
  if (x == 0.0 || isnan(x) || isinf(x)) return x;
  int e;
  frexp(x, &e);
  int q = e - 11;                /* exponent of the last kept bit */
  if (q < -24) q = -24;          /* subnormal binary16 quantum */
  double r = ldexp(rint(ldexp(x, -q)), q);
  if (fabs(r) > 65504.0) r = copysign(INFINITY, x);
  return r;
}

/* Round a double to binary32, ties to even (C conversion in the default rounding mode). */
double orc_round_f32(double x) { return (double)(float)x; }

/* Storage types of a table: 0 binary32, 1 bfloat16, 2 binary16 (the C ABI's dtype codes). */
static double round_store(double x, int32_t stype) {
  return stype == 1 ? orc_round_bf16(x) : stype == 2 ? orc_round_f16(x) : orc_round_f32(x);
}

/* ------------------------------------------------------------------ table fill */
/* splitmix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014): the state advances by the golden-ratio increment, and the output is the
 * state passed through two xor-shift-multiply rounds and a final xor-shift. */
uint64_t orc_splitmix64_next(uint64_t* state) {
  uint64_t z = (*state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Table element (global_row, col): one splitmix64 output from state seed ^ (row*dim+col);
 * its top 24 bits give u in [0,1); x = fp32(2u-1) * fp32(1/sqrt(rows_t)) in binary32;
 * bf16 and fp16 storage (stype 1, 2) round x to nearest-even.  Returns the stored value. */
double orc_table_value(uint64_t seed, int64_t global_row, int64_t col, int32_t dim,
                       int64_t rows_t, int32_t stype) {
  uint64_t st = seed ^ (uint64_t)(global_row * (int64_t)dim + col);
  uint64_t v = orc_splitmix64_next(&st);
  double u = (double)(v >> 40) * (1.0 / 16777216.0);
  float a = (float)(1.0 / sqrt((double)rows_t));
  float s = (float)(2.0 * u - 1.0);
  float x = s * a;
  return round_store((double)x, stype);
}

typedef struct {
  const float* data;        /* host copy of the table values, or NULL: regenerate */
  uint64_t seed;
  const int64_t* row_base;  /* [num_tables + 1] */
  int32_t num_tables;
  int32_t dim;
  int32_t stype;            /* storage type: 0 binary32, 1 bfloat16, 2 binary16 */
} orc_table;

static int64_t rows_of_key(const orc_table* tb, int64_t key) {
  for (int32_t t = 0; t < tb->num_tables; ++t)
    if (key >= tb->row_base[t] && key < tb->row_base[t + 1])
      return tb->row_base[t + 1] - tb->row_base[t];
  return -1;
}

static double tval(const orc_table* tb, int64_t key, int64_t col) {
  if (tb->data) return (double)tb->data[key * (int64_t)tb->dim + col];
  return orc_table_value(tb->seed, key, col, tb->dim, rows_of_key(tb, key), tb->stype);
}

/* Fill rows `keys[0..n)` of the described table into out[n][dim] (as stored values). */
void orc_table_rows(uint64_t seed, const int64_t* row_base, int32_t num_tables, int32_t dim,
                    int32_t stype, const int64_t* keys, int64_t n, float* out) {
  orc_table tb = {NULL, seed, row_base, num_tables, dim, stype};
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r)
    for (int64_t c = 0; c < dim; ++c) out[r * dim + c] = (float)tval(&tb, keys[r], c);
}

/* ------------------------------------------------------------------ a1: keys */
/* key[i] = row_base[t] + (modulus > 0 ? floor_mod(id[i], modulus) : id[i]) for the
 * occurrence i inside bag (t, b), bags table-major with `batch` bags per table. */
void orc_form_keys(const int64_t* ids, const int64_t* offsets, int64_t num_tables,
                   int64_t batch, const int64_t* row_base, int64_t modulus, int64_t* keys) {
  for (int64_t t = 0; t < num_tables; ++t)
    for (int64_t b = 0; b < batch; ++b) {
      int64_t s = t * batch + b;
      for (int64_t i = offsets[s]; i < offsets[s + 1]; ++i) {
        int64_t id = ids[i];
        if (modulus > 0) {
          id %= modulus;
          if (id < 0) id += modulus;
        }
        keys[i] = (row_base ? row_base[t] : 0) + id;
      }
    }
}

/* ------------------------------------------------------------------ a2: unique */
typedef struct {
  int64_t key;
  int64_t idx;
} kv;

static int kv_cmp(const void* a, const void* b) {
  const kv* x = (const kv*)a;
  const kv* y = (const kv*)b;
  if (x->key != y->key) return x->key < y->key ? -1 : 1;
  return x->idx < y->idx ? -1 : (x->idx > y->idx);
}

/* [TN] "Core Optimizations": sort the batch's IDs and give each distinct ID a contiguous
 * index.  Sorting (key, occurrence) pairs makes the order total, hence stable.
 *   uniq[u]      distinct keys, ascending (signed)
 *   inverse[i]   u with uniq[u] == key[i]
 *   perm[p]      occurrence at sorted position p (stable argsort)
 *   seg[u]       first sorted position of uniq[u]; seg[U] = n
 * Returns U. */
int64_t orc_unique(const int64_t* keys, int64_t n, int64_t* uniq, int32_t* inverse,
                   int32_t* perm, int32_t* seg) {
  if (n == 0) {
    if (seg) seg[0] = 0;
    return 0;
  }
  kv* a = (kv*)malloc((size_t)n * sizeof(kv));
  for (int64_t i = 0; i < n; ++i) {
    a[i].key = keys[i];
    a[i].idx = i;
  }
  qsort(a, (size_t)n, sizeof(kv), kv_cmp);
  int64_t u = -1;
  for (int64_t p = 0; p < n; ++p) {
    if (p == 0 || a[p].key != a[p - 1].key) {
      ++u;
      uniq[u] = a[p].key;
      if (seg) seg[u] = (int32_t)p;
    }
    inverse[a[p].idx] = (int32_t)u;
    if (perm) perm[p] = (int32_t)a[p].idx;
  }
  if (seg) seg[u + 1] = (int32_t)n;
  free(a);
  return u + 1;
}

/* ------------------------------------------------------------------ a3: gather */
/* [TN] "Core Optimizations": fetch the batch's rows into the batch-sized matrix,
 * E[u] = W[rows[u]]. */
void orc_gather_rows(const float* data, uint64_t seed, const int64_t* row_base,
                     int32_t num_tables, int32_t dim, int32_t stype, const int64_t* rows,
                     int64_t n, double* out) {
  orc_table tb = {data, seed, row_base, num_tables, dim, stype};
#pragma omp parallel for schedule(static)
  for (int64_t u = 0; u < n; ++u)
    for (int64_t c = 0; c < dim; ++c) out[u * dim + c] = tval(&tb, rows[u], c);
}

/* ------------------------------------------------------------------ a4: pooling */
/* [DHEN] 2.1: one d-dim vector per sparse feature.  Sum pooling of the bag's rows (each
 * occurrence counted, empty bag = 0).  out and mag are [batch][num_tables][dim].
 * Row of occurrence i: key = row_base[t] + ids[i] (ids are table-local rows here). */
void orc_embbag_fwd(const float* data, uint64_t seed, const int64_t* row_base,
                    int32_t num_tables, int32_t dim, int32_t stype, const int64_t* ids,
                    const int64_t* offsets, int64_t batch, double* out, double* mag) {
  orc_table tb = {data, seed, row_base, num_tables, dim, stype};
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t s = 0; s < (int64_t)num_tables * batch; ++s) {
    int64_t t = s / batch, b = s % batch;
    double* o = out + (b * num_tables + t) * dim;
    double* m = mag + (b * num_tables + t) * dim;
    for (int64_t c = 0; c < dim; ++c) {
      o[c] = 0.0;
      m[c] = 0.0;
    }
    for (int64_t i = offsets[s]; i < offsets[s + 1]; ++i) {
      int64_t key = row_base[t] + ids[i];
      for (int64_t c = 0; c < dim; ++c) {
        double w = tval(&tb, key, c);
        o[c] += w;
        m[c] += fabs(w);
      }
    }
  }
}

/* ------------------------------------------------------------------ a6: interaction */
/* A factor of a pair product: the value itself, or (bf16 != 0) the value rounded to bf16
 * nearest-even.  The bf16 form is the reading taken for workloads whose tables are stored in
 * bf16 with fp32 accumulation: the interaction's operands (Z, and the pair gradients in the
 * backward) are rounded to bf16 once, their products and sums are exact here. */
static double operand(double x, int32_t bf16) { return bf16 ? orc_round_bf16(x) : x; }

/* [DLRM] 02 and [DHEN] 3.1 / Solution 2: for each sample, the dense vector z_0 followed by
 * the dot products <z_i, z_j> of every pair i > j (strict: C(F,2) of them), in the order
 * of the row-major strict lower triangle, index i(i-1)/2 + j.  The dense part of R is z_0
 * as it is (a copy, never rounded).
 * Z, zmag: [batch][F][dim] (zmag may be NULL: the absolute values of the factors);
 * R, rmag: [batch][dim + P]; bf16: factors rounded to bf16 (operand() above). */
void orc_interaction_fwd(const double* Z, const double* zmag, int64_t batch, int32_t F,
                         int32_t dim, int32_t bf16, double* R, double* rmag) {
  int64_t P = (int64_t)F * (F - 1) / 2, W = dim + P;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < batch; ++b) {
    const double* z = Z + b * F * dim;
    const double* zm = zmag ? zmag + b * F * dim : NULL;
    for (int64_t c = 0; c < dim; ++c) {
      R[b * W + c] = z[c];
      rmag[b * W + c] = zm ? zm[c] : fabs(z[c]);
    }
    for (int64_t i = 1; i < F; ++i)
      for (int64_t j = 0; j < i; ++j) {
        double s = 0.0, a = 0.0;
        for (int64_t c = 0; c < dim; ++c) {
          double xi = operand(z[i * dim + c], bf16), xj = operand(z[j * dim + c], bf16);
          s += xi * xj;
          double mi = zm ? zm[i * dim + c] : fabs(xi);
          double mj = zm ? zm[j * dim + c] : fabs(xj);
          a += mi * mj;
        }
        R[b * W + dim + i * (i - 1) / 2 + j] = s;
        rmag[b * W + dim + i * (i - 1) / 2 + j] = a;
      }
  }
}

/* ------------------------------------------------------------------ a7: its gradient */
/* Chain rule of the interaction above: with dP_ij the upstream gradient of pair (i, j),
 * dZ_i = sum over j != i of dP_(max(i,j), min(i,j)) * z_j, and the upstream gradient of
 * the dense passthrough adds to dZ_0.  dR: [batch][dim + P]; dZ, dmag: [batch][F][dim].
 * bf16: dP and z_j rounded to bf16 (operand()); the dense passthrough's gradient is added as
 * it is. */
void orc_interaction_bwd(const double* Z, const double* zmag, const double* dR,
                         int64_t batch, int32_t F, int32_t dim, int32_t bf16, double* dZ,
                         double* dmag) {
  int64_t P = (int64_t)F * (F - 1) / 2, W = dim + P;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < batch; ++b) {
    const double* z = Z + b * F * dim;
    const double* zm = zmag ? zmag + b * F * dim : NULL;
    const double* g = dR + b * W;
    for (int64_t i = 0; i < F; ++i)
      for (int64_t c = 0; c < dim; ++c) {
        double s = 0.0, a = 0.0;
        for (int64_t j = 0; j < F; ++j) {
          if (j == i) continue;
          int64_t hi = i > j ? i : j, lo = i > j ? j : i;
          double gp = operand(g[dim + hi * (hi - 1) / 2 + lo], bf16);
          double zj = operand(z[j * dim + c], bf16);
          s += gp * zj;
          a += fabs(gp) * (zm ? zm[j * dim + c] : fabs(zj));
        }
        if (i == 0) {
          s += g[c];
          a += fabs(g[c]);
        }
        dZ[(b * F + i) * dim + c] = s;
        dmag[(b * F + i) * dim + c] = a;
      }
  }
}

/* ------------------------------------------------------------------ a8: row gradients */
/* Chain rule of sum pooling: every occurrence in bag (t, b) receives dY[b][t]; the rows'
 * gradients are those summed per distinct row, in the order of uniq ([TN] "Synchronous
 * Architecture": only rows present in the batch get a gradient).  No 1/B scaling.
 * dY, dymag: [batch][num_tables][dim]; inverse from orc_unique; g, gmag: [U][dim]. */
void orc_embbag_bwd(const double* dY, const double* dymag, const int64_t* offsets,
                    int64_t batch, int32_t num_tables, int32_t dim, const int32_t* inverse,
                    int64_t U, double* g, double* gmag) {
  memset(g, 0, (size_t)U * dim * sizeof(double));
  memset(gmag, 0, (size_t)U * dim * sizeof(double));
  for (int64_t t = 0; t < num_tables; ++t)
    for (int64_t b = 0; b < batch; ++b) {
      int64_t s = t * batch + b;
      const double* y = dY + (b * num_tables + t) * dim;
      const double* ym = dymag ? dymag + (b * num_tables + t) * dim : NULL;
      for (int64_t i = offsets[s]; i < offsets[s + 1]; ++i) {
        int64_t u = inverse[i];
        for (int64_t c = 0; c < dim; ++c) {
          g[u * dim + c] += y[c];
          gmag[u * dim + c] += ym ? ym[c] : fabs(y[c]);
        }
      }
    }
}

/* ------------------------------------------------------------------ a9: sparse SGD */
/* W[uniq[u]] <- W[uniq[u]] - lr * g[u] in double, rounded once to the storage type
 * (binary32, or bfloat16 / binary16 nearest-even).  Rows not in uniq are untouched by definition.
 * new_rows, nmag: [U][dim] (nmag = |W| + lr * gmag). */
void orc_sparse_sgd(const float* data, uint64_t seed, const int64_t* row_base,
                    int32_t num_tables, int32_t dim, int32_t stype, const int64_t* uniq,
                    int64_t U, const double* g, const double* gmag, float lr,
                    double* new_rows, double* nmag) {
  orc_table tb = {data, seed, row_base, num_tables, dim, stype};
  double l = (double)lr;
#pragma omp parallel for schedule(static)
  for (int64_t u = 0; u < U; ++u)
    for (int64_t c = 0; c < dim; ++c) {
      double w = tval(&tb, uniq[u], c);
      double x = w - l * g[u * dim + c];
      new_rows[u * dim + c] = round_store(x, stype);
      nmag[u * dim + c] = fabs(w) + l * gmag[u * dim + c];
    }
}

/* ------------------------------------------------------------------ interaction variants */
/* [DHEN] 3.1: all inner products <x_i, x_j> for i <= j, self-dots included.  Pairs i >= j of
 * z_0..z_{F-1} in row-major lower-triangle order, index i(i+1)/2 + j; R = [z_0 | pairs],
 * P = F(F+1)/2.  Magnitudes and the bf16 factors as in orc_interaction_fwd. */
void orc_interaction_self_fwd(const double* Z, const double* zmag, int64_t batch, int32_t F,
                              int32_t dim, int32_t bf16, double* R, double* rmag) {
  int64_t P = (int64_t)F * (F + 1) / 2, W = dim + P;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < batch; ++b) {
    const double* z = Z + b * F * dim;
    const double* zm = zmag ? zmag + b * F * dim : NULL;
    for (int64_t c = 0; c < dim; ++c) {
      R[b * W + c] = z[c];
      rmag[b * W + c] = zm ? zm[c] : fabs(z[c]);
    }
    for (int64_t i = 0; i < F; ++i)
      for (int64_t j = 0; j <= i; ++j) {
        double s = 0.0, a = 0.0;
        for (int64_t c = 0; c < dim; ++c) {
          double xi = operand(z[i * dim + c], bf16), xj = operand(z[j * dim + c], bf16);
          s += xi * xj;
          double mi = zm ? zm[i * dim + c] : fabs(xi);
          double mj = zm ? zm[j * dim + c] : fabs(xj);
          a += mi * mj;
        }
        R[b * W + dim + i * (i + 1) / 2 + j] = s;
        rmag[b * W + dim + i * (i + 1) / 2 + j] = a;
      }
  }
}

/* Chain rule of the pair set with self-dots: dZ_i = sum over j != i of dP_(max,min) z_j
 * + 2 dP_ii z_i (the derivative of <z_i, z_i>), plus the dense passthrough's gradient on
 * dZ_0.  dR: [batch][dim + F(F+1)/2]; bf16 as in orc_interaction_bwd (the doubled self
 * term is 2 times the rounded dP_ii). */
void orc_interaction_self_bwd(const double* Z, const double* zmag, const double* dR,
                              int64_t batch, int32_t F, int32_t dim, int32_t bf16, double* dZ,
                              double* dmag) {
  int64_t P = (int64_t)F * (F + 1) / 2, W = dim + P;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < batch; ++b) {
    const double* z = Z + b * F * dim;
    const double* zm = zmag ? zmag + b * F * dim : NULL;
    const double* g = dR + b * W;
    for (int64_t i = 0; i < F; ++i)
      for (int64_t c = 0; c < dim; ++c) {
        double s = 0.0, a = 0.0;
        for (int64_t j = 0; j < F; ++j) {
          int64_t hi = i > j ? i : j, lo = i > j ? j : i;
          double gp = operand(g[dim + hi * (hi + 1) / 2 + lo], bf16);
          double zj = operand(z[j * dim + c], bf16);
          double k = (j == i) ? 2.0 : 1.0;
          s += k * gp * zj;
          a += k * fabs(gp) * (zm ? zm[j * dim + c] : fabs(zj));
        }
        if (i == 0) {
          s += g[c];
          a += fabs(g[c]);
        }
        dZ[(b * F + i) * dim + c] = s;
        dmag[(b * F + i) * dim + c] = a;
      }
  }
}

/* [DHEN] 3.3, eq. (7): a DCN-style layer takes the whole Gram matrix X X^T of a sample's
 * vectors.  R[b][dim + i F + j] = <z_i, z_j> for all i, j < F (row-major, both triangles and
 * the diagonal), after the dense slot R[b][0 .. dim) = z_0.  Magnitudes and the bf16 factors
 * as in orc_interaction_fwd.  R, rmag: [batch][dim + F F]. */
void orc_interaction_gram_fwd(const double* Z, const double* zmag, int64_t batch, int32_t F,
                              int32_t dim, int32_t bf16, double* R, double* rmag) {
  int64_t P = (int64_t)F * F, W = dim + P;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < batch; ++b) {
    const double* z = Z + b * F * dim;
    const double* zm = zmag ? zmag + b * F * dim : NULL;
    for (int64_t c = 0; c < dim; ++c) {
      R[b * W + c] = z[c];
      rmag[b * W + c] = zm ? zm[c] : fabs(z[c]);
    }
    for (int64_t i = 0; i < F; ++i)
      for (int64_t j = 0; j < F; ++j) {
        double s = 0.0, a = 0.0;
        for (int64_t c = 0; c < dim; ++c) {
          double xi = operand(z[i * dim + c], bf16), xj = operand(z[j * dim + c], bf16);
          s += xi * xj;
          double mi = zm ? zm[i * dim + c] : fabs(xi);
          double mj = zm ? zm[j * dim + c] : fabs(xj);
          a += mi * mj;
        }
        R[b * W + dim + i * F + j] = s;
        rmag[b * W + dim + i * F + j] = a;
      }
  }
}

/* Chain rule of the Gram matrix: <z_i, z_j> sits at (i, j) and (j, i), so
 * dZ_i = sum over j of (dG_ij + dG_ji) z_j (on the diagonal 2 dG_ii z_i), plus the dense
 * passthrough's gradient on dZ_0.  Without bf16 the factor S_ij = dG_ij + dG_ji is exact here;
 * with bf16 != 0 it is formed as a matrix-core kernel takes it, the binary32 sum of the two
 * binary32 gradients rounded to bf16 (the reading for bf16 workloads, orc_interaction_bwd), and
 * z_j is rounded to bf16; products and sums stay exact.  Magnitude per term:
 * (|dG_ij| + |dG_ji|) |z_j| (|S_ij| |z_j| with bf16).  dR: [batch][dim + F F]. */
void orc_interaction_gram_bwd(const double* Z, const double* zmag, const double* dR,
                              int64_t batch, int32_t F, int32_t dim, int32_t bf16, double* dZ,
                              double* dmag) {
  int64_t P = (int64_t)F * F, W = dim + P;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < batch; ++b) {
    const double* z = Z + b * F * dim;
    const double* zm = zmag ? zmag + b * F * dim : NULL;
    const double* g = dR + b * W + dim;
    for (int64_t i = 0; i < F; ++i)
      for (int64_t c = 0; c < dim; ++c) {
        double s = 0.0, a = 0.0;
        for (int64_t j = 0; j < F; ++j) {
          double gij = g[i * F + j], gji = g[j * F + i];
          double sij, mij;
          if (bf16) {
            float s32 = (float)gij + (float)gji;          /* binary32 sum, one rounding */
            sij = orc_round_bf16((double)s32);
            mij = fabs(sij);
          } else {
            sij = gij + gji;
            mij = fabs(gij) + fabs(gji);
          }
          double zj = operand(z[j * dim + c], bf16);
          s += sij * zj;
          a += mij * (zm ? zm[j * dim + c] : fabs(zj));
        }
        if (i == 0) {
          s += dR[b * W + c];
          a += fabs(dR[b * W + c]);
        }
        dZ[(b * F + i) * dim + c] = s;
        dmag[(b * F + i) * dim + c] = a;
      }
  }
}

/* [DHEN] Solution 2, the FM sum: out[b] = sum over F > i > j >= 0 of <z_i, z_j>, written as
 * that definition (O(F^2 d)).  The magnitude also counts 1/2 sum_i ||z_i||^2: the O(F d)
 * squared-norm form 1/2 (||sum z_i||^2 - sum ||z_i||^2) cancels those self terms, and a
 * forward-error bound of that evaluation scales with them. */
void orc_fm_fwd(const double* Z, const double* zmag, int64_t batch, int32_t F, int32_t dim,
                double* out, double* omag) {
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < batch; ++b) {
    const double* z = Z + b * F * dim;
    const double* zm = zmag ? zmag + b * F * dim : NULL;
    double s = 0.0, a = 0.0;
    for (int64_t i = 0; i < F; ++i)
      for (int64_t j = 0; j <= i; ++j)
        for (int64_t c = 0; c < dim; ++c) {
          double mi = zm ? zm[i * dim + c] : fabs(z[i * dim + c]);
          double mj = zm ? zm[j * dim + c] : fabs(z[j * dim + c]);
          if (j < i) {
            s += z[i * dim + c] * z[j * dim + c];
            a += mi * mj;
          } else {
            a += 0.5 * mi * mj;
          }
        }
    out[b] = s;
    omag[b] = a;
  }
}

/* Its gradient: dZ_i = dout[b] * sum over j != i of z_j.  The magnitude sums |z_j| over all
 * j (the O(F d) form computes sum_j z_j - z_i). */
void orc_fm_bwd(const double* Z, const double* zmag, const double* dout, int64_t batch,
                int32_t F, int32_t dim, double* dZ, double* dmag) {
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < batch; ++b) {
    const double* z = Z + b * F * dim;
    const double* zm = zmag ? zmag + b * F * dim : NULL;
    for (int64_t i = 0; i < F; ++i)
      for (int64_t c = 0; c < dim; ++c) {
        double s = 0.0, a = 0.0;
        for (int64_t j = 0; j < F; ++j) {
          double m = zm ? zm[j * dim + c] : fabs(z[j * dim + c]);
          if (j != i) s += z[j * dim + c];
          a += m;
        }
        dZ[(b * F + i) * dim + c] = dout[b] * s;
        dmag[(b * F + i) * dim + c] = fabs(dout[b]) * a;
      }
  }
}

/* ------------------------------------------------------------------ dense layers, head */
/* [DLRM] 02 "Arquitetura": the continuous features pass through a bottom MLP whose output is
 * the dense vector of the interaction; the interaction's output passes through a top MLP
 * and a sigmoid that gives the click probability.  One fully connected layer, written from
 * its definition: Y[m][n] = act(b[n] + sum_k X[m][k] W[n][k]), act = ReLU (max(., 0)) or the
 * identity.  X [M][K], W [N][K], b [N] or NULL, Y [M][N].  bf16: each product takes X and W
 * rounded to bf16 nearest-even (the bias is added as it is).  Xm: magnitudes of X (NULL:
 * |X|); Ym = |b| + sum |x| |w|. */
void orc_dense_fwd(const double* X, const double* Xm, int64_t M, int32_t K, const double* W,
                   const double* b, int32_t N, int32_t relu, int32_t bf16, double* Y,
                   double* Ym) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double s = b ? b[n] : 0.0, a = b ? fabs(b[n]) : 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double x = X[m * K + k], w = W[n * K + k];
        if (bf16) {
          x = orc_round_bf16(x);
          w = orc_round_bf16(w);
        }
        s += x * w;
        a += (Xm ? Xm[m * K + k] : fabs(x)) * fabs(w);
      }
      Y[m * N + n] = (relu && !(s > 0.0)) ? 0.0 : s;
      Ym[m * N + n] = a;
    }
}

/* The layer's backward and the SGD step of its parameters, by the chain rule on the
 * definition above with the gradients summed over the M rows:
 *   dA[m][n] = dY[m][n] if the layer is linear or Y[m][n] > 0, else 0
 *   dX[m][k] = sum_n dA[m][n] W[n][k]
 *   W'[n][k] = W[n][k] - lr sum_m dA[m][n] X[m][k]
 *   b'[n]    = b[n] - lr sum_m dA[m][n]
 * bf16: dA, W and X are rounded to bf16 nearest-even in the products; the bias is the weight
 * of a constant input 1, so its sum takes the same rounded dA.  W' and b' are rounded once to
 * binary32, the stored parameter type.
 * Magnitudes: dXm = sum |dA| |W|, Wm = |W| + lr sum |dA| |X|, bm = |b| + lr sum |dA|.
 * dX, b, bn may be NULL. */
void orc_dense_bwd_sgd(const double* X, int64_t M, int32_t K, const double* W, const double* b,
                       int32_t N, int32_t relu, const double* Y, const double* dY, int32_t bf16,
                       double lr, double* dX, double* dXm, double* Wn, double* Wm, double* bn,
                       double* bm) {
  double* dA = (double*)malloc(sizeof(double) * (size_t)(M * N > 0 ? M * N : 1));
  for (int64_t i = 0; i < M * N; ++i) dA[i] = (relu && !(Y[i] > 0.0)) ? 0.0 : dY[i];
  if (dX) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
      for (int64_t k = 0; k < K; ++k) {
        double s = 0.0, a = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          double g = dA[m * N + n], w = W[n * K + k];
          if (bf16) {
            g = orc_round_bf16(g);
            w = orc_round_bf16(w);
          }
          s += g * w;
          a += fabs(g) * fabs(w);
        }
        dX[m * K + k] = s;
        dXm[m * K + k] = a;
      }
  }
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t k = 0; k < K; ++k) {
      double s = 0.0, a = 0.0;
      for (int64_t m = 0; m < M; ++m) {
        double g = dA[m * N + n], x = X[m * K + k];
        if (bf16) {
          g = orc_round_bf16(g);
          x = orc_round_bf16(x);
        }
        s += g * x;
        a += fabs(g) * fabs(x);
      }
      Wn[n * K + k] = orc_round_f32(W[n * K + k] - lr * s);
      Wm[n * K + k] = fabs(W[n * K + k]) + lr * a;
    }
    if (b && bn) {
      double s = 0.0, a = 0.0;
      for (int64_t m = 0; m < M; ++m) {
        const double g = bf16 ? orc_round_bf16(dA[m * N + n]) : dA[m * N + n];
        s += g;
        a += fabs(g);
      }
      bn[n] = orc_round_f32(b[n] - lr * s);
      bm[n] = fabs(b[n]) + lr * a;
    }
  }
  free(dA);
}

/* The logistic head and normalized entropy.  [DLRM] 02: a sigmoid gives the click
 * probability p = 1 / (1 + e^-s).  [DHEN] 7.1 "Setup": NE = (mean binary cross-entropy) /
 * H(q), q the empirical click rate of the labels, H(q) = -(q ln q + (1-q) ln(1-q));
 * Solution 17: the cross-entropy of a logit is softplus(s) - y s, here
 * (max(s, 0) - y s) + log1p(e^-|s|).  Per element: prob, the gradient of the mean
 * cross-entropy (p - y) / M and its magnitude (p + |y|) / M.  stats = [sum ce, sum y, NE]
 * (NE is NaN when q is 0 or 1); stats_mag = [sum |terms of ce|, sum |y|, NE magnitude
 * (sum |terms| / M / H(q))]. */
void orc_logistic_ne(const double* s, const double* y, int64_t M, double* prob, double* dl,
                     double* dlm, double* stats, double* stats_mag) {
  double sce = 0.0, sy = 0.0, ace = 0.0, ay = 0.0;
  for (int64_t i = 0; i < M; ++i) {
    const double x = s[i], l = y[i];
    const double p = 1.0 / (1.0 + exp(-x));
    const double sp = log1p(exp(-fabs(x)));
    sce += (fmax(x, 0.0) - l * x) + sp;
    ace += fabs(fmax(x, 0.0)) + fabs(l * x) + sp;
    sy += l;
    ay += fabs(l);
    prob[i] = p;
    dl[i] = (p - l) / (double)M;
    dlm[i] = (p + fabs(l)) / (double)M;
  }
  const double q = sy / (double)M;
  const double h = -(q * log(q) + (1.0 - q) * log(1.0 - q));
  stats[0] = sce;
  stats[1] = sy;
  stats[2] = (q > 0.0 && q < 1.0) ? (sce / (double)M) / h : NAN;
  stats_mag[0] = ace;
  stats_mag[1] = ay;
  stats_mag[2] = (q > 0.0 && q < 1.0) ? (ace / (double)M) / h : NAN;
}

/* ------------------------------------------------------------------ exported dictionary */
/* [TN] "Inference Optimization": online inference looks raw IDs up in a pre-exported sparse
 * embedding dictionary.  The dictionary is the list (keys[e], rows[e], hot[e]) of its n
 * entries; the value of ID x is ((hot[e] + 1) << 32) | rows[e] for the entry with
 * keys[e] == x, or -1 when there is none (negative IDs have none).  Written as a search
 * over the entries sorted by key (`order`, a permutation the caller gets from a library
 * sort), one binary search per ID. */
void orc_dict_lookup(const int64_t* keys, const int32_t* rows, const int32_t* hot,
                     const int64_t* order, int64_t n, const int64_t* ids, int64_t m,
                     int64_t* values) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; ++i) {
    int64_t x = ids[i], lo = 0, hi = n, v = -1;
    while (lo < hi) {                              /* first sorted entry with key >= x */
      int64_t mid = lo + (hi - lo) / 2;
      if (keys[order[mid]] < x) lo = mid + 1; else hi = mid;
    }
    if (x >= 0 && lo < n && keys[order[lo]] == x) {
      int64_t e = order[lo];
      uint64_t hs = hot ? (uint64_t)(uint32_t)(hot[e] + 1) : 0u;
      v = (int64_t)((hs << 32) | (uint32_t)rows[e]);
    }
    values[i] = v;
  }
}

/* Sum pooling over looked-up values: out[b][t][c] = sum over the bag's occurrences with
 * values[k] >= 0 of W[row][c], row = the low 32 bits of values[k] (the cache holds copies
 * of dictionary rows, so the cached or the table copy is the same value).  W is the
 * dictionary table (one table of num_rows rows, the counter-based fill or `data`). */
void orc_dict_pool(const float* data, uint64_t seed, int64_t num_rows, int32_t dim,
                   int32_t stype, const int64_t* values, const int64_t* offsets, int64_t batch,
                   int32_t num_tables, double* out, double* omag) {
  int64_t rb[2] = {0, num_rows};
  orc_table tb = {data, seed, rb, 1, dim, stype};
  int64_t nb = (int64_t)num_tables * batch;
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < nb; ++s) {
    int64_t t = s / batch, b = s - t * batch;
    double* o = out + (b * num_tables + t) * dim;
    double* om = omag + (b * num_tables + t) * dim;
    for (int64_t c = 0; c < dim; ++c) {
      o[c] = 0.0;
      om[c] = 0.0;
    }
    for (int64_t k = offsets[s]; k < offsets[s + 1]; ++k) {
      if (values[k] < 0) continue;
      int64_t row = (int64_t)(uint32_t)values[k];
      if (row >= num_rows) continue;
      for (int64_t c = 0; c < dim; ++c) {
        double w = tval(&tb, row, c);
        o[c] += w;
        om[c] += fabs(w);
      }
    }
  }
}

/* ------------------------------------------------------------------ stochastic rounding */
/* [DHEN] 6.4 names stochastic rounding for low-precision embedding updates and gives no
 * formula; the textbook definition is taken, for bfloat16 storage.  x lies between the
 * adjacent bfloat16 values lo (toward zero) and hi = lo + sign(x) * quantum (away from
 * zero); SR(x) = hi with probability p = (|x| - |lo|) / quantum, else lo.  The probability
 * is realised by a uniform 16-bit integer r: hi iff r < p * 2^16.  For a binary32 x, p is
 * a multiple of 2^-16, so over all 2^16 values of r the mean of SR(x) is exactly x.
 * Exact values (p = 0), zeros, infinities and NaN come back unchanged; a value above the
 * largest finite bfloat16 that rounds up becomes infinity. */
double orc_sr_bf16(double x, uint32_t r) {
  if (x == 0.0 || isnan(x) || isinf(x)) return x;
  int e;
  frexp(x, &e);
  int q = e - 8;                 /* exponent of the last kept bit, as in orc_round_bf16 */
  if (q < -133) q = -133;
  double quantum = ldexp(1.0, q);
  double lo = ldexp(trunc(ldexp(x, -q)), q);
  double p = (fabs(x) - fabs(lo)) / quantum;       /* exact, in [0, 1) */
  double out = ((double)r < p * 65536.0) ? lo + copysign(quantum, x) : lo;
  if (fabs(out) > 3.3895313892515355e38) out = copysign(INFINITY, x);
  return out;
}

/* The same rule for binary16 storage ("DHEN" notes, 6.4: FP16 embeddings with stochastic
 * rounding): lo is x truncated toward zero to binary16 (11 significant bits, quantum no finer
 * than 2^-24), hi iff r < p * 2^16.  Here p can carry more than 16 bits (13 bits are dropped
 * in the normal range, up to 125 below it), so SR(x) averages to x plus at most quantum *
 * 2^-16 over the 2^16 values of r: the comparison rounds the probability up to a multiple of
 * 2^-16.  Zeros, infinities and NaN come back unchanged; anything whose result exceeds the
 * largest finite binary16, 65504, becomes infinity (so |x| >= 65536 always does). */
double orc_sr_f16(double x, uint32_t r) {
  if (x == 0.0 || isnan(x) || isinf(x)) return x;
  int e;
  frexp(x, &e);
  int q = e - 11;                /* exponent of the last kept bit, as in orc_round_f16 */
  if (q < -24) q = -24;
  double quantum = ldexp(1.0, q);
  double lo = ldexp(trunc(ldexp(x, -q)), q);
  double p = (fabs(x) - fabs(lo)) / quantum;       /* exact, in [0, 1) */
  double out = ((double)r < p * 65536.0) ? lo + copysign(quantum, x) : lo;
  if (fabs(out) > 65504.0) out = copysign(INFINITY, x);
  return out;
}

/* Random bits of element (key, col) of an update drawn with seed s: columns are taken in
 * groups of four, c4 = col - col mod 4; one splitmix64 output from state s ^ (key*dim + c4)
 * (the same generator as the table fill, a fresh seed per update) gives 64 bits, and
 * column c4 + e takes bits 16e .. 16e+15 of it. */
uint32_t orc_sr_bits(uint64_t seed, int64_t key, int64_t col, int32_t dim) {
  int64_t e = col % 4;
  uint64_t st = seed ^ (uint64_t)(key * (int64_t)dim + (col - e));
  return (uint32_t)((orc_splitmix64_next(&st) >> (16 * e)) & 0xFFFFu);
}

/* a9 with stochastic rounding, bfloat16 (stype 1) or binary16 (stype 2) storage:
 * W[uniq[u]] <- SR(x) with x = fmaf(-lr, g[u], W[uniq[u]]), the binary32 fused multiply-add
 * rounded once.  The value that decides the rounding is taken in binary32, the precision the
 * update kernel computes in (g is binary32 here).  new_rows: [U][dim]. */
void orc_sparse_sgd_sr(const float* data, uint64_t seed, const int64_t* row_base,
                       int32_t num_tables, int32_t dim, int32_t stype, const int64_t* uniq,
                       int64_t U, const float* g, float lr, uint64_t sr_seed, double* new_rows) {
  orc_table tb = {data, seed, row_base, num_tables, dim, stype};
#pragma omp parallel for schedule(static)
  for (int64_t u = 0; u < U; ++u)
    for (int64_t c = 0; c < dim; ++c) {
      float w = (float)tval(&tb, uniq[u], c);
      float x = fmaf(-lr, g[u * dim + c], w);
      uint32_t r = orc_sr_bits(sr_seed, uniq[u], c, dim);
      new_rows[u * dim + c] = stype == 2 ? orc_sr_f16((double)x, r) : orc_sr_bf16((double)x, r);
    }
}
