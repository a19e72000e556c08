// prepare.hip -- COO validation, segment offsets and load-balanced tiles (gfx950).
//
// The tiles cut the merge path of segment ends and entries (Merrill &
// Garland, "Merge-based Parallel Sparse Matrix-Vector Multiplication", SC'16)
// every T items, then move each cut back to the start of its segment unless
// that segment holds >= T entries.  Every tile thus carries < 2T items, short
// rows are never split, and only long rows spill across tiles -- the answer
// to the imbalance described in "Two Lotteries: What It Takes to Make
// Sparsity Fast" (paragraph on who does the work).
//
// Both kernels here are single passes over sorted data with no searches:
// offsets are written where the sorted key changes, and the cuts are
// enumerated per segment (segment s owns path items ptr[s]+s .. ptr[s+1]+s,
// so the cuts inside it are the multiples of T in that range).  Every write
// is clamped to its array, so an invalid COO is reported through `err`
// without any out-of-bounds access.
#include "common.h"
#include "internal.h"

namespace snk {

constexpr int PREP_THREADS = 256;

// ptr[r] = first position k whose key is >= r, for r in [0, S], from keys
// sorted ascending: thread k writes ptr[r] = k for key[k-1] < r <= key[k];
// thread nnz closes the trailing segments with nnz.  With `col` non-NULL the
// keys are the COO rows and the COO is validated: err bit 0 = index out of
// range, bit 1 = not strictly increasing in row*K + col.
__global__ __launch_bounds__(PREP_THREADS) void k_seg_bounds(const int32_t* __restrict__ keys,
                                                             const int32_t* __restrict__ col,
                                                             int64_t nnz, int32_t S, int32_t K,
                                                             int32_t* __restrict__ ptr,
                                                             int32_t* __restrict__ err) {
  const int64_t k = (int64_t)blockIdx.x * PREP_THREADS + threadIdx.x;
  if (k > nnz) return;
  const int64_t prev = k > 0 ? (int64_t)keys[k - 1] : -1;
  const int64_t key = k < nnz ? (int64_t)keys[k] : (int64_t)S;
  const int64_t lo = std::max<int64_t>(prev + 1, 0), hi = std::min<int64_t>(key, S);
  for (int64_t r = lo; r <= hi; ++r) ptr[r] = (int32_t)k;
  if (col && k < nnz) {
    const int32_t c = col[k];
    int32_t bits = 0;
    if (key < 0 || key >= S || c < 0 || c >= K) bits |= 1;
    if (k > 0) {
      const int64_t lin = key * K + c;
      const int64_t plin = prev * K + col[k - 1];
      if (lin <= plin) bits |= 2;
    }
    if (bits) atomicOr(err, bits);
  }
}

// Tile start points, enumerated per segment.  Cut p (at item p*T) that falls
// on segment s is (s, p*T - s) if s is long (>= T entries) and the cut is
// past its first entry -- an "inner" cut, cut[p] = 1 -- else (s, ptr[s]).
// Thread S writes the closing point (S, nnz).  any_split is set when an inner
// cut exists.
__global__ __launch_bounds__(PREP_THREADS) void k_tiles(const int32_t* __restrict__ ptr,
                                                        int32_t S, int64_t nnz, int32_t T,
                                                        int32_t P, int32_t* __restrict__ part_seg,
                                                        int32_t* __restrict__ part_nz,
                                                        int32_t* __restrict__ cut,
                                                        int32_t* __restrict__ any_split) {
  const int64_t s = (int64_t)blockIdx.x * PREP_THREADS + threadIdx.x;
  if (s > S) return;
  if (s == S) {
    part_seg[P] = S;
    part_nz[P] = (int32_t)nnz;
    cut[P] = 0;
    return;
  }
  const int64_t a = ptr[s], b = ptr[s + 1];
  if (a < 0 || b < a || b > nnz) return;  // invalid COO: reported by k_seg_bounds
  const int64_t first = a + s, last = b + s;
  const int64_t p0 = (first + T - 1) / T;
  const int64_t p1 = std::min<int64_t>(last / T, (int64_t)P - 1);
  const bool is_long = (b - a) >= T;
  bool any = false;
  for (int64_t p = p0; p <= p1; ++p) {
    const int64_t z = p * T - s;
    const bool inner = is_long && z != a;
    part_seg[p] = (int32_t)s;
    part_nz[p] = (int32_t)(inner ? z : a);
    cut[p] = inner ? 1 : 0;
    any |= inner;
  }
  if (any) atomicOr(any_split, 1);
}

static inline dim3 grid_for(int64_t n) {
  return dim3((unsigned)std::max<int64_t>(1, cdiv(n, PREP_THREADS)));
}

hipError_t launch_seg_bounds(const int32_t* keys, const int32_t* col, int64_t nnz, int32_t S,
                             int32_t K, int32_t* ptr, int32_t* err, hipStream_t s) {
  hipLaunchKernelGGL(k_seg_bounds, grid_for(nnz + 1), dim3(PREP_THREADS), 0, s, keys, col, nnz,
                     S, K, ptr, err);
  return hipGetLastError();
}

hipError_t launch_tiles(const int32_t* ptr, int32_t S, int64_t nnz, int32_t T, int32_t P,
                        int32_t* part_seg, int32_t* part_nz, int32_t* cut, int32_t* any_split,
                        hipStream_t s) {
  hipLaunchKernelGGL(k_tiles, grid_for((int64_t)S + 1), dim3(PREP_THREADS), 0, s, ptr, S, nnz, T,
                     P, part_seg, part_nz, cut, any_split);
  return hipGetLastError();
}

}  // namespace snk
