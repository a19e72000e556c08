/*
 * oracle.c -- plain, serial, fp64 CPU oracle for the truly sparse linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant generator with the HIP library: it is written
 * from the definitions alone, for a reader to check by eye.
 *
 * What the layer computes ("Beyond Masked Sparsity: SNACK Enables Truly
 * Sparse Neural Networks on GPU", Abstract): a layer that stores and computes
 * only its nonzero connections, in COO form, with the backward pass kept in
 * the sparse form as well.  With W an M x K matrix (out x in) whose nonzeros
 * are (row[k], col[k], v[k]), strictly increasing in row*K + col:
 *
 *   forward        Y[b, r]  = sum_{k : row[k] = r} v[k] * X[b, col[k]]
 *   input grad     dX[b, c] = sum_{k : col[k] = c} v[k] * dY[b, row[k]]
 *   value grad     dV[k]    = sum_b dY[b, row[k]] * X[b, col[k]]
 *
 * i.e. Y = X W^T, dX = dY W and dV = (dY^T X) sampled at the nonzeros.  All
 * sums are accumulated in double, one term at a time, in increasing k (or b)
 * order.  Alongside each output the oracle returns the magnitude scale
 * S = sum |term|, against which a float result is judged.
 *
 * Activations are either batch-major (X[b*F + f]) or node-major (X[f*B + b]).
 *
 * Parity pins (see tests/test_oracle_pins.py): a dense masked product through
 * numpy, the identities dX = dY W_dense and dV = (dY^T X)[row, col], the
 * error scales against the same products taken over |W|, |X| and |dY|, the
 * adjoint identity <dY, Y> = <dX, X> = <v, dV>, exact finite differences of
 * a bilinear map, brute-force recounts of the derived index arrays, a full
 * lexicographic sort for the prune, and published SplitMix64 outputs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_E_RANGE (-5)
#define ORC_E_ORDER (-6)
#define ORC_E_NAN (-7)
#define ORC_E_COUNT (-8)
#define ORC_E_NOMEM (-12)

static inline int64_t aidx(int64_t b, int64_t f, int64_t B, int64_t F, int node_major) {
  return node_major ? f * B + b : b * F + f;
}

/* ---------------------------------------------------------------- checks */
int orc_validate_coo(int32_t M, int32_t K, int64_t nnz, const int32_t* row, const int32_t* col) {
  int64_t prev = -1;
  for (int64_t k = 0; k < nnz; ++k) {
    if (row[k] < 0 || row[k] >= M || col[k] < 0 || col[k] >= K) return ORC_E_RANGE;
  }
  for (int64_t k = 0; k < nnz; ++k) {
    int64_t lin = (int64_t)row[k] * K + col[k];
    if (lin <= prev) return ORC_E_ORDER;
    prev = lin;
  }
  return ORC_OK;
}

/* ------------------------------------------------------------- products */
void orc_spmm_fwd(int32_t M, int32_t K, int64_t nnz, const int32_t* row, const int32_t* col,
                  const double* v, int32_t B, const double* X, int node_major, double* Y,
                  double* S) {
  memset(Y, 0, sizeof(double) * (size_t)B * M);
  if (S) memset(S, 0, sizeof(double) * (size_t)B * M);
  for (int64_t k = 0; k < nnz; ++k) {
    for (int32_t b = 0; b < B; ++b) {
      double t = v[k] * X[aidx(b, col[k], B, K, node_major)];
      int64_t o = aidx(b, row[k], B, M, node_major);
      Y[o] += t;
      if (S) S[o] += fabs(t);
    }
  }
}

void orc_spmm_bwd_input(int32_t M, int32_t K, int64_t nnz, const int32_t* row,
                        const int32_t* col, const double* v, int32_t B, const double* dY,
                        int node_major, double* dX, double* S) {
  memset(dX, 0, sizeof(double) * (size_t)B * K);
  if (S) memset(S, 0, sizeof(double) * (size_t)B * K);
  for (int64_t k = 0; k < nnz; ++k) {
    for (int32_t b = 0; b < B; ++b) {
      double t = v[k] * dY[aidx(b, row[k], B, M, node_major)];
      int64_t o = aidx(b, col[k], B, K, node_major);
      dX[o] += t;
      if (S) S[o] += fabs(t);
    }
  }
}

void orc_sddmm(int32_t M, int32_t K, int64_t nnz, const int32_t* row, const int32_t* col,
               int32_t B, const double* dY, const double* X, int node_major, double* dV,
               double* S) {
  for (int64_t k = 0; k < nnz; ++k) {
    double acc = 0.0, mag = 0.0;
    for (int32_t b = 0; b < B; ++b) {
      double t = dY[aidx(b, row[k], B, M, node_major)] * X[aidx(b, col[k], B, K, node_major)];
      acc += t;
      mag += fabs(t);
    }
    dV[k] = acc;
    if (S) S[k] = mag;
  }
}

/* exact-erf GELU and its derivative (aux op between the two MLP layers) */
void orc_gelu(int64_t n, const double* z, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = 0.5 * z[i] * (1.0 + erf(z[i] / sqrt(2.0)));
}

void orc_gelu_bwd(int64_t n, const double* z, const double* dy, double* out) {
  const double inv_sqrt_2pi = 0.39894228040143267794;
  for (int64_t i = 0; i < n; ++i) {
    double cdf = 0.5 * (1.0 + erf(z[i] / sqrt(2.0)));
    double pdf = inv_sqrt_2pi * exp(-0.5 * z[i] * z[i]);
    out[i] = dy[i] * (cdf + z[i] * pdf);
  }
}

/* ------------------------------------------------ derived index arrays */
/* Row-segment offsets: count the entries of every row, then prefix-sum. */
void orc_row_ptr(int32_t M, int64_t nnz, const int32_t* row, int32_t* row_ptr) {
  memset(row_ptr, 0, sizeof(int32_t) * ((size_t)M + 1));
  for (int64_t k = 0; k < nnz; ++k) row_ptr[row[k] + 1] += 1;
  for (int32_t r = 0; r < M; ++r) row_ptr[r + 1] += row_ptr[r];
}

/* Column view by a stable counting sort on col: perm[i] is the row-major
 * position of the i-th entry in (col, row) order, row_t[i] = row[perm[i]]. */
int orc_csc(int32_t K, int64_t nnz, const int32_t* row, const int32_t* col, int32_t* col_ptr,
            int32_t* perm, int32_t* row_t) {
  memset(col_ptr, 0, sizeof(int32_t) * ((size_t)K + 1));
  for (int64_t k = 0; k < nnz; ++k) col_ptr[col[k] + 1] += 1;
  for (int32_t c = 0; c < K; ++c) col_ptr[c + 1] += col_ptr[c];
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * ((size_t)K + 1));
  if (!cursor) return ORC_E_NOMEM;
  memcpy(cursor, col_ptr, sizeof(int32_t) * ((size_t)K + 1));
  for (int64_t k = 0; k < nnz; ++k) {
    int32_t i = cursor[col[k]]++;
    perm[i] = (int32_t)k;
    row_t[i] = row[k];
  }
  free(cursor);
  return ORC_OK;
}

/*
 * Load-balanced partition of a segmented stream (rows of the row view, or
 * columns of the column view) into tiles of about T work items.
 *
 * The work of S segments with offsets ptr[0..S] is the sequence of items
 * obtained by listing, for each segment in turn, its L_s = ptr[s+1]-ptr[s]
 * entries followed by one "segment end" item: I = S + nnz items in all (the
 * merge path of the segment ends with the entries, Merrill & Garland,
 * "Merge-based Parallel Sparse Matrix-Vector Multiplication", SC'16).  A
 * point on it is (s, z): s segment ends and z entries consumed.  Item
 * positions of segment s run from ptr[s]+s to ptr[s+1]+s (its end item).
 *
 * Tile p nominally starts at item d = p*T, p = 0..P-1, P = ceil(I/T); the
 * boundary after the last tile is (S, nnz).  If d falls on segment s:
 *   - at the first entry of s (z = ptr[s]) the boundary is (s, ptr[s]);
 *   - otherwise, if s is short (L_s < T), the boundary moves back to the
 *     start of s, (s, ptr[s]): short segments are never split;
 *   - otherwise (L_s >= T) the boundary is (s, d - s), inside s.
 *
 * A segment is "split" when a boundary (s, z) with z > ptr[s] lies in it.
 * For every split segment, in increasing s, the oracle lists (s, p_first,
 * p_last): the tile holding its first entry and the tile holding its end.
 *
 * Returns P; fills part_seg/part_nz[0..P] and the split list (returns its
 * length through *n_split).  This is a serial sweep over the segments.
 */
int64_t orc_partition(int32_t S, int64_t nnz, const int32_t* ptr, int64_t T, int32_t* part_seg,
                      int32_t* part_nz, int32_t* split_seg, int32_t* split_first,
                      int32_t* split_last, int64_t* n_split) {
  int64_t I = (int64_t)S + nnz;
  int64_t P = (I + T - 1) / T;
  int64_t ns = 0;
  for (int32_t s = 0; s < S; ++s) {
    int64_t L = (int64_t)ptr[s + 1] - ptr[s];
    int64_t first_pos = (int64_t)ptr[s] + s;      /* position of its first item */
    int64_t end_pos = (int64_t)ptr[s + 1] + s;    /* position of its end item */
    /* multiples of T in [first_pos, end_pos] */
    int64_t p0 = (first_pos + T - 1) / T;
    int64_t p_inner_first = -1, p_inner_last = -1;
    for (int64_t p = p0; p * T <= end_pos && p < P; ++p) {
      int64_t d = p * T;
      int64_t z = d - s;
      if (z == ptr[s]) {
        part_seg[p] = s;
        part_nz[p] = ptr[s];
      } else if (L < T) {
        part_seg[p] = s;
        part_nz[p] = ptr[s];
      } else {
        part_seg[p] = s;
        part_nz[p] = (int32_t)z;
        if (p_inner_first < 0) p_inner_first = p;
        p_inner_last = p;
      }
    }
    if (p_inner_first >= 0) {
      split_seg[ns] = s;
      split_first[ns] = (int32_t)(p_inner_first - 1);
      split_last[ns] = (int32_t)p_inner_last;
      ++ns;
    }
  }
  part_seg[P] = S;
  part_nz[P] = (int32_t)nnz;
  *n_split = ns;
  return P;
}

/* --------------------------------------------------------- prune/regrow */
/* SplitMix64 (Steele, Lea & Flood, "Fast Splittable Pseudorandom Number
 * Generators", OOPSLA 2014): the state advances by the golden gamma, and each
 * output is the state passed through the variant-13 finaliser. */
static const uint64_t SM_GAMMA = 0x9E3779B97F4A7C15ULL;

static uint64_t sm_finalise(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* i-th output (i = 0, 1, ...) of a generator seeded with `state`. */
uint64_t orc_splitmix64(uint64_t state, uint64_t i) {
  return sm_finalise(state + (i + 1) * SM_GAMMA);
}

/* n_drop = round half up of nnz * ppm / 1e6 */
int64_t orc_drop_count(int64_t nnz, int32_t ppm) {
  return (int64_t)(((__int128)nnz * ppm + 500000) / 1000000);
}

typedef struct {
  uint32_t mag;
  int64_t lin;
  int64_t k;
} orc_key;

static int cmp_key(const void* a, const void* b) {
  const orc_key* x = (const orc_key*)a;
  const orc_key* y = (const orc_key*)b;
  if (x->mag != y->mag) return x->mag < y->mag ? -1 : 1;
  if (x->lin != y->lin) return x->lin < y->lin ? -1 : 1;
  return 0;
}

static int cmp_i64(const void* a, const void* b) {
  int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
  return x < y ? -1 : (x > y ? 1 : 0);
}

static int in_sorted(const int64_t* a, int64_t n, int64_t x) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    int64_t mid = lo + (hi - lo) / 2;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo < n && a[lo] == x;
}

/* open-addressing set of int64 >= 0 */
typedef struct {
  int64_t* slot;
  int64_t cap;
} orc_set;

static int set_insert(orc_set* h, int64_t x) { /* 1 if newly inserted */
  uint64_t i = sm_finalise((uint64_t)x) & (uint64_t)(h->cap - 1);
  while (h->slot[i] >= 0) {
    if (h->slot[i] == x) return 0;
    i = (i + 1) & (uint64_t)(h->cap - 1);
  }
  h->slot[i] = x;
  return 1;
}

/*
 * One prune-and-regrow step of dynamic sparse training on a COO weight
 * ("restructuring connections", Abstract of the SNACK page).  The page names
 * the operation but not its rule; the rule implemented here is:
 *
 * 1. NaN values are an error.  Magnitude key of entry k: its value's bit
 *    pattern with the sign bit cleared (so -0 == +0), fp32 or bf16 bits.
 * 2. The n_drop entries smallest in (magnitude key, linear index row*K+col)
 *    are dropped; survivors keep their values and order.
 * 3. Regrowth: stream state s = SplitMix64 output number `step` of a
 *    generator seeded with `seed`; candidate i = 0,1,... is
 *    p_i = floor(x_i * (M*K) / 2^64) with x_i output number i of a generator
 *    seeded with s.  p_i is accepted if it is not in the pre-step support and
 *    was not accepted before; the first n_drop acceptances are grown.
 * 4. New support = survivors + grown, sorted by linear index; grown values
 *    are 0 (bit pattern 0).
 *
 * dropped_lin / grown_lin (nullable) receive the dropped and grown linear
 * indices in increasing order.  vbits holds fp32 bits, or bf16 bits in the
 * low 16 bits when is_bf16.
 */
int orc_prune_regrow(int32_t M, int32_t K, int64_t nnz, const int32_t* row, const int32_t* col,
                     const uint32_t* vbits, int is_bf16, int64_t n_drop, uint64_t seed,
                     uint64_t step, int32_t* out_row, int32_t* out_col, uint32_t* out_vbits,
                     int64_t* dropped_lin, int64_t* grown_lin) {
  const int64_t MK = (int64_t)M * K;
  if (n_drop < 0 || n_drop > nnz || n_drop > MK - nnz) return ORC_E_COUNT;
  for (int64_t k = 0; k < nnz; ++k) {
    uint32_t a = is_bf16 ? (vbits[k] & 0x7FFFu) : (vbits[k] & 0x7FFFFFFFu);
    if (is_bf16 ? (a > 0x7F80u) : (a > 0x7F800000u)) return ORC_E_NAN;
  }
  int64_t* support = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nnz + 1));
  orc_key* keys = (orc_key*)malloc(sizeof(orc_key) * (size_t)(nnz + 1));
  char* dropped = (char*)calloc((size_t)nnz + 1, 1);
  int64_t* grown = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_drop + 1));
  if (!support || !keys || !dropped || !grown) {
    free(support); free(keys); free(dropped); free(grown);
    return ORC_E_NOMEM;
  }
  for (int64_t k = 0; k < nnz; ++k) {
    support[k] = (int64_t)row[k] * K + col[k];
    keys[k].mag = is_bf16 ? (vbits[k] & 0x7FFFu) : (vbits[k] & 0x7FFFFFFFu);
    keys[k].lin = support[k];
    keys[k].k = k;
  }
  qsort(keys, (size_t)nnz, sizeof(orc_key), cmp_key);
  for (int64_t i = 0; i < n_drop; ++i) dropped[keys[i].k] = 1;

  /* regrowth stream */
  int64_t cap = 16;
  while (cap < 4 * (n_drop + 1)) cap <<= 1;
  orc_set acc = {(int64_t*)malloc(sizeof(int64_t) * (size_t)cap), cap};
  if (!acc.slot) {
    free(support); free(keys); free(dropped); free(grown);
    return ORC_E_NOMEM;
  }
  for (int64_t i = 0; i < cap; ++i) acc.slot[i] = -1;
  uint64_t s = orc_splitmix64(seed, step);
  int64_t got = 0;
  for (uint64_t i = 0; got < n_drop; ++i) {
    uint64_t x = orc_splitmix64(s, i);
    int64_t p = (int64_t)(uint64_t)(((unsigned __int128)x * (uint64_t)MK) >> 64);
    if (in_sorted(support, nnz, p)) continue;
    if (!set_insert(&acc, p)) continue;
    grown[got++] = p;
  }
  qsort(grown, (size_t)n_drop, sizeof(int64_t), cmp_i64);

  /* merge survivors (already increasing) with grown (sorted) */
  int64_t i = 0, j = 0, o = 0, nd = 0;
  while (i < nnz || j < n_drop) {
    if (i < nnz && dropped[i]) {
      if (dropped_lin) dropped_lin[nd] = support[i];
      ++nd;
      ++i;
      continue;
    }
    int take_survivor = (j >= n_drop) || (i < nnz && support[i] < grown[j]);
    int64_t lin = take_survivor ? support[i] : grown[j];
    out_row[o] = (int32_t)(lin / K);
    out_col[o] = (int32_t)(lin % K);
    out_vbits[o] = take_survivor ? vbits[i] : 0u;
    ++o;
    if (take_survivor) ++i; else ++j;
  }
  if (grown_lin) memcpy(grown_lin, grown, sizeof(int64_t) * (size_t)n_drop);
  free(acc.slot);
  free(support);
  free(keys);
  free(dropped);
  free(grown);
  return ORC_OK;
}
