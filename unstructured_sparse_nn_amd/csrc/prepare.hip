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
// Both main kernels here are single passes over sorted data with no searches:
// offsets are written where the sorted key changes, and the cuts are
// enumerated per segment (segment s owns path items ptr[s]+s .. ptr[s+1]+s,
// so the cuts inside it are the multiples of T in that range).  Every write
// is clamped to its array, so an invalid COO is reported through the
// per-block error flags without any out-of-bounds access.
#include "common.h"
#include "internal.h"
#include "results.h"
#include "tiles.h"

namespace snk {

constexpr int PREP_THREADS = 256;

// ptr[r] = first position k whose key is >= r, for r in [0, S], from keys
// sorted ascending: thread k writes ptr[r] = k for key[k-1] < r <= key[k];
// thread nnz closes the trailing segments with nnz.  With `col` non-NULL the
// keys are the COO rows and the COO is validated: errs[block] receives the
// OR of its threads' bits (bit 0 = index out of range, bit 1 = not strictly
// increasing in row*K + col), written by every block (no zeroing needed).
__global__ __launch_bounds__(PREP_THREADS) void k_seg_bounds(const int32_t* __restrict__ keys,
                                                             const int32_t* __restrict__ col,
                                                             int64_t nnz, int32_t S, int32_t K,
                                                             int32_t* __restrict__ ptr,
                                                             int32_t* __restrict__ errs) {
  const int64_t k = (int64_t)blockIdx.x * PREP_THREADS + threadIdx.x;
  int32_t bits = 0;
  if (k <= nnz) {
    const int64_t prev = k > 0 ? (int64_t)keys[k - 1] : -1;
    const int64_t key = k < nnz ? (int64_t)keys[k] : (int64_t)S;
    const int64_t lo = std::max<int64_t>(prev + 1, 0), hi = std::min<int64_t>(key, S);
    for (int64_t r = lo; r <= hi; ++r) ptr[r] = (int32_t)k;
    if (col && k < nnz) {
      const int32_t c = col[k];
      if (key < 0 || key >= S || c < 0 || c >= K) bits |= 1;
      if (k > 0) {
        const int64_t lin = key * K + c;
        const int64_t plin = prev * K + col[k - 1];
        if (lin <= plin) bits |= 2;
      }
    }
  }
  if (errs) {
    __shared__ int32_t w_or[PREP_THREADS / SNK_WAVE];
    for (int off = 32; off > 0; off >>= 1) bits |= __shfl_xor(bits, off, SNK_WAVE);
    if (lane_id() == 0) w_or[threadIdx.x / SNK_WAVE] = bits;
    __syncthreads();
    if (threadIdx.x == 0) {
      int32_t b = 0;
      for (int i = 0; i < PREP_THREADS / SNK_WAVE; ++i) b |= w_or[i];
      errs[blockIdx.x] = b;
    }
  }
}

// Tile start points, enumerated per segment (tile_cuts); thread S writes
// the closing point (S, nnz).  splits[block] = 1 if one of the block's
// segments has an inner cut (written by every block).
__global__ __launch_bounds__(PREP_THREADS) void k_tiles(const int32_t* __restrict__ ptr,
                                                        int32_t S, int64_t nnz, int32_t T,
                                                        int32_t P, int32_t* __restrict__ part_seg,
                                                        int32_t* __restrict__ part_nz,
                                                        int32_t* __restrict__ cut,
                                                        int32_t* __restrict__ splits) {
  const int64_t s = (int64_t)blockIdx.x * PREP_THREADS + threadIdx.x;
  bool any = false;
  if (s == S) tile_close(S, nnz, P, part_seg, part_nz, cut);
  else if (s < S) any = tile_cuts(s, ptr[s], ptr[s + 1], nnz, T, P, part_seg, part_nz, cut);
  const int b = __syncthreads_or(any ? 1 : 0);
  if (threadIdx.x == 0) splits[blockIdx.x] = b ? 1 : 0;
}

// One workgroup: OR of the per-block flags of prepare, written straight into
// pinned host memory: res[0] = error bits, res[1] / res[2] = the row / column
// view has a segment split across tiles.
constexpr int RES_THREADS = 1024;
__device__ __forceinline__ int32_t block_or(int32_t v, int32_t* lds) {
  for (int off = 32; off > 0; off >>= 1) v |= __shfl_xor(v, off, SNK_WAVE);
  if (lane_id() == 0) lds[threadIdx.x / SNK_WAVE] = v;
  __syncthreads();
  int32_t o = 0;
  for (int i = 0; i < RES_THREADS / SNK_WAVE; ++i) o |= lds[i];
  __syncthreads();
  return o;
}

__global__ __launch_bounds__(RES_THREADS) void k_prepare_result(
    const int32_t* __restrict__ errs, int64_t n_errs, const int32_t* __restrict__ rsplit,
    int64_t n_r, const int32_t* __restrict__ csplit, int64_t n_c, int32_t* __restrict__ res) {
  __shared__ int32_t lds[RES_THREADS / SNK_WAVE];
  int32_t e = 0, r = 0, c = 0;
  for (int64_t i = threadIdx.x; i < n_errs; i += RES_THREADS) e |= errs[i];
  for (int64_t i = threadIdx.x; i < n_r; i += RES_THREADS) r |= rsplit[i];
  for (int64_t i = threadIdx.x; i < n_c; i += RES_THREADS) c |= csplit[i];
  e = block_or(e, lds);
  r = block_or(r, lds);
  c = block_or(c, lds);
  if (threadIdx.x == 0) {
    store_result(&res[0], e);
    store_result(&res[1], r);
    store_result(&res[2], c);
  }
}

static inline dim3 grid_for(int64_t n) {
  return dim3((unsigned)std::max<int64_t>(1, cdiv(n, PREP_THREADS)));
}

int64_t seg_bounds_blocks(int64_t nnz) { return std::max<int64_t>(1, cdiv(nnz + 1, PREP_THREADS)); }
int64_t tiles_blocks(int32_t S) { return std::max<int64_t>(1, cdiv((int64_t)S + 1, PREP_THREADS)); }

hipError_t launch_seg_bounds(const int32_t* keys, const int32_t* col, int64_t nnz, int32_t S,
                             int32_t K, int32_t* ptr, int32_t* errs, hipStream_t s) {
  hipLaunchKernelGGL(k_seg_bounds, grid_for(nnz + 1), dim3(PREP_THREADS), 0, s, keys, col, nnz,
                     S, K, ptr, errs);
  return hipGetLastError();
}

hipError_t launch_tiles(const int32_t* ptr, int32_t S, int64_t nnz, int32_t T, int32_t P,
                        int32_t* part_seg, int32_t* part_nz, int32_t* cut, int32_t* splits,
                        hipStream_t s) {
  hipLaunchKernelGGL(k_tiles, grid_for((int64_t)S + 1), dim3(PREP_THREADS), 0, s, ptr, S, nnz, T,
                     P, part_seg, part_nz, cut, splits);
  return hipGetLastError();
}

hipError_t launch_prepare_result(const int32_t* errs, int64_t n_errs, const int32_t* rsplit,
                                 int64_t n_r, const int32_t* csplit, int64_t n_c, int32_t* res,
                                 hipStream_t s) {
  hipLaunchKernelGGL(k_prepare_result, dim3(1), dim3(RES_THREADS), 0, s, errs, n_errs, rsplit,
                     n_r, csplit, n_c, res);
  return hipGetLastError();
}

}  // namespace snk
