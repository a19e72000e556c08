// tiles.h -- the load-balanced tile cuts of one segment (device helper
// shared by prepare and by the fused restructure).
//
// The tiles cut the merge path of segment ends and entries (Merrill &
// Garland, "Merge-based Parallel Sparse Matrix-Vector Multiplication", SC'16)
// every T items; each cut moves back to the start of its segment unless that
// segment holds >= T entries.  Segment s owns path items a+s .. b+s (entries
// [a, b)), so the cuts inside it are the multiples of T in that range.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace snk {

// Writes the tile start points that fall on segment s: cut p (item p*T) is
// (s, p*T - s) if s is long and the cut is past its first entry -- an
// "inner" cut, cut[p] = 1 -- else (s, a).  Returns true if an inner cut was
// written.  Does nothing for an inconsistent range (a < 0, b < a, b > nnz).
__device__ __forceinline__ bool tile_cuts(int64_t s, int64_t a, int64_t b, int64_t nnz,
                                          int32_t T, int32_t P, int32_t* __restrict__ part_seg,
                                          int32_t* __restrict__ part_nz,
                                          int32_t* __restrict__ cut) {
  if (a < 0 || b < a || b > nnz) return false;
  const int64_t first = a + s, last = b + s;
  int64_t p0, pl;
  if (last + T <= (int64_t)UINT32_MAX) {  // 32-bit division when the items fit
    p0 = ((uint32_t)first + (uint32_t)T - 1u) / (uint32_t)T;
    pl = (uint32_t)last / (uint32_t)T;
  } else {
    p0 = (first + T - 1) / T;
    pl = last / T;
  }
  const int64_t p1 = std::min<int64_t>(pl, (int64_t)P - 1);
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
  return any;
}

// The closing point (S, nnz) of a view with S segments and P tiles.
__device__ __forceinline__ void tile_close(int32_t S, int64_t nnz, int32_t P,
                                           int32_t* __restrict__ part_seg,
                                           int32_t* __restrict__ part_nz,
                                           int32_t* __restrict__ cut) {
  part_seg[P] = S;
  part_nz[P] = (int32_t)nnz;
  cut[P] = 0;
}

}  // namespace snk
