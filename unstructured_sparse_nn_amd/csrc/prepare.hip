// prepare.hip -- COO validation, segment offsets, load-balanced tiles (gfx950).
//
// The tiles cut the merge path of segment ends and entries (Merrill &
// Garland, "Merge-based Parallel Sparse Matrix-Vector Multiplication", SC'16)
// every T items, then move each cut back to the start of its segment unless
// that segment holds >= T entries.  Every tile thus carries < 2T items, short
// rows are never split, and only long rows spill across tiles -- the answer
// to the imbalance described in "Two Lotteries: What It Takes to Make
// Sparsity Fast" (paragraph on who does the work).
#include "common.h"
#include "internal.h"

namespace snk {

constexpr int PREP_THREADS = 256;

// err bit 0: index out of range; bit 1: not strictly increasing.
__global__ __launch_bounds__(PREP_THREADS) void k_validate(const int32_t* __restrict__ row,
                                                           const int32_t* __restrict__ col,
                                                           int64_t nnz, int32_t M, int32_t K,
                                                           int32_t* __restrict__ err) {
  int64_t k = (int64_t)blockIdx.x * PREP_THREADS + threadIdx.x;
  if (k >= nnz) return;
  int32_t r = row[k], c = col[k];
  int32_t bits = 0;
  if (r < 0 || r >= M || c < 0 || c >= K) bits |= 1;
  if (k > 0) {
    int64_t lin = (int64_t)r * K + c;
    int64_t prev = (int64_t)row[k - 1] * K + col[k - 1];
    if (lin <= prev) bits |= 2;
  }
  if (bits) atomicOr(err, bits);
}

// ptr[s] = first position whose key is >= s, for s in [0, S] (keys sorted).
__global__ __launch_bounds__(PREP_THREADS) void k_seg_ptr(const int32_t* __restrict__ keys,
                                                          int64_t nnz, int32_t S,
                                                          int32_t* __restrict__ ptr) {
  int64_t s = (int64_t)blockIdx.x * PREP_THREADS + threadIdx.x;
  if (s > S) return;
  int64_t lo = 0, hi = nnz;
  while (lo < hi) {
    int64_t mid = (lo + hi) >> 1;
    if (keys[mid] < s) lo = mid + 1; else hi = mid;
  }
  ptr[s] = (int32_t)lo;
}

// Tile start points.  Segment s owns path items ptr[s]+s .. ptr[s+1]+s (its
// entries, then its end); the segment holding item d = p*T is the number of
// segments whose end item lies before d.
__global__ __launch_bounds__(PREP_THREADS) void k_partition(const int32_t* __restrict__ ptr,
                                                            int32_t S, int64_t nnz, int32_t T,
                                                            int32_t P,
                                                            int32_t* __restrict__ part_seg,
                                                            int32_t* __restrict__ part_nz) {
  int64_t p = (int64_t)blockIdx.x * PREP_THREADS + threadIdx.x;
  if (p > P) return;
  if (p == P) {
    part_seg[p] = S;
    part_nz[p] = (int32_t)nnz;
    return;
  }
  int64_t d = p * (int64_t)T;
  int64_t lo = 0, hi = S;  // count of t with ptr[t+1] + t < d
  while (lo < hi) {
    int64_t mid = (lo + hi) >> 1;
    if ((int64_t)ptr[mid + 1] + mid < d) lo = mid + 1; else hi = mid;
  }
  int32_t s = (int32_t)lo;
  int64_t z = d - s;
  int32_t a = ptr[s], b = ptr[s + 1];
  if (z != a && (b - a) < T) z = a;
  part_seg[p] = s;
  part_nz[p] = (int32_t)z;
}

__device__ __forceinline__ bool inner_cut(const int32_t* ptr, const int32_t* ps,
                                          const int32_t* pz, int64_t p, int32_t P) {
  if (p <= 0 || p >= P) return false;
  return pz[p] > ptr[ps[p]];
}

// first[p] = 1 if tile p's start is the first cut inside a split segment.
__global__ __launch_bounds__(PREP_THREADS) void k_split_flags(const int32_t* __restrict__ ptr,
                                                              const int32_t* __restrict__ ps,
                                                              const int32_t* __restrict__ pz,
                                                              int32_t P,
                                                              int32_t* __restrict__ first) {
  int64_t p = (int64_t)blockIdx.x * PREP_THREADS + threadIdx.x;
  if (p >= P) return;
  bool in = inner_cut(ptr, ps, pz, p, P);
  bool prev_same = in && inner_cut(ptr, ps, pz, p - 1, P) && ps[p - 1] == ps[p];
  first[p] = (in && !prev_same) ? 1 : 0;
}

// Split j: (segment, tile holding its first entry, tile holding its end).
__global__ __launch_bounds__(PREP_THREADS) void k_split_write(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ ps,
    const int32_t* __restrict__ pz, int32_t P, const int32_t* __restrict__ first,
    const int32_t* __restrict__ scan, int32_t* __restrict__ split) {
  int64_t p = (int64_t)blockIdx.x * PREP_THREADS + threadIdx.x;
  if (p >= P) return;
  if (!inner_cut(ptr, ps, pz, p, P)) return;
  int32_t j = scan[p] + first[p] - 1;
  if (first[p]) {
    split[3 * j + 0] = ps[p];
    split[3 * j + 1] = (int32_t)(p - 1);
  }
  bool next_same = inner_cut(ptr, ps, pz, p + 1, P) && ps[p + 1] == ps[p];
  if (!next_same) split[3 * j + 2] = (int32_t)p;
}

__global__ __launch_bounds__(PREP_THREADS) void k_gather_i32(const int32_t* __restrict__ src,
                                                             const int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ dst,
                                                             int64_t n) {
  int64_t i = (int64_t)blockIdx.x * PREP_THREADS + threadIdx.x;
  if (i < n) dst[i] = src[idx[i]];
}

__global__ __launch_bounds__(PREP_THREADS) void k_iota_i32(int32_t* __restrict__ dst, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * PREP_THREADS + threadIdx.x;
  if (i < n) dst[i] = (int32_t)i;
}

static inline dim3 grid_for(int64_t n) {
  return dim3((unsigned)std::max<int64_t>(1, cdiv(n, PREP_THREADS)));
}

hipError_t launch_validate(const int32_t* row, const int32_t* col, int64_t nnz, int32_t M,
                           int32_t K, int32_t* err, hipStream_t s) {
  if (nnz > 0)
    hipLaunchKernelGGL(k_validate, grid_for(nnz), dim3(PREP_THREADS), 0, s, row, col, nnz, M, K,
                       err);
  return hipGetLastError();
}

hipError_t launch_seg_ptr(const int32_t* keys, int64_t nnz, int32_t S, int32_t* ptr,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_seg_ptr, grid_for((int64_t)S + 1), dim3(PREP_THREADS), 0, s, keys, nnz,
                     S, ptr);
  return hipGetLastError();
}

hipError_t launch_partition(const int32_t* ptr, int32_t S, int64_t nnz, int32_t T, int32_t P,
                            int32_t* part_seg, int32_t* part_nz, int32_t* flags_first,
                            int32_t* flags_scan, int32_t* split, int32_t* n_split_dev,
                            void* scan_tmp, hipStream_t s) {
  hipLaunchKernelGGL(k_partition, grid_for((int64_t)P + 1), dim3(PREP_THREADS), 0, s, ptr, S,
                     nnz, T, P, part_seg, part_nz);
  if (P > 0) {
    hipLaunchKernelGGL(k_split_flags, grid_for(P), dim3(PREP_THREADS), 0, s, ptr, part_seg,
                       part_nz, P, flags_first);
  }
  hipError_t e = exclusive_scan_i32(flags_first, flags_scan, P, n_split_dev, scan_tmp, s);
  if (e != hipSuccess) return e;
  if (P > 0) {
    hipLaunchKernelGGL(k_split_write, grid_for(P), dim3(PREP_THREADS), 0, s, ptr, part_seg,
                       part_nz, P, flags_first, flags_scan, split);
  }
  return hipGetLastError();
}

hipError_t launch_gather_i32(const int32_t* src, const int32_t* idx, int32_t* dst, int64_t n,
                             hipStream_t s) {
  if (n > 0)
    hipLaunchKernelGGL(k_gather_i32, grid_for(n), dim3(PREP_THREADS), 0, s, src, idx, dst, n);
  return hipGetLastError();
}

hipError_t launch_iota_i32(int32_t* dst, int64_t n, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(k_iota_i32, grid_for(n), dim3(PREP_THREADS), 0, s, dst, n);
  return hipGetLastError();
}

}  // namespace snk
