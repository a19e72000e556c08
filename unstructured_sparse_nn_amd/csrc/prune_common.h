// prune_common.h -- pieces shared by the two device plans of prune/regrow.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/snack.h"

namespace snk {

// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): the state advances by the
// golden gamma; an output is the variant-13 mix of the state.
__host__ __device__ __forceinline__ uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
constexpr uint64_t SM64_GAMMA = 0x9E3779B97F4A7C15ull;

// Grid position of stream candidate i: output i of a generator seeded with
// `stream` (= state stream + (i+1) gamma), scaled to [0, MK) by the high
// half of the 128-bit product (Lemire's multiply-shift, no rejection).
__device__ __forceinline__ uint64_t sm64_position(uint64_t stream, uint64_t i, uint64_t MK) {
  return __umul64hi(sm64_mix(stream + (i + 1) * SM64_GAMMA), MK);
}

__device__ __forceinline__ int64_t cdiv_dev(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Magnitude key of a value: its bits with the sign cleared (-0 == +0).
template <typename T>
__device__ __forceinline__ uint32_t raw_bits(T v) {
  if constexpr (sizeof(T) == 4) return __float_as_uint(v);
  else return (uint32_t)v;
}
template <typename T>
__device__ __forceinline__ uint32_t magnitude(uint32_t bits) {
  return sizeof(T) == 2 ? (bits & 0x7FFFu) : (bits & 0x7FFFFFFFu);
}
template <typename T>
__device__ __forceinline__ bool is_nan_mag(uint32_t a) {
  return sizeof(T) == 2 ? (a > 0x7F80u) : (a > 0x7F800000u);
}

// ---- plan choice (prune.hip) ----------------------------------------------------
// The bitmap plan when it applies, unless flags has SNACK_PRUNE_SORT_PLAN.
bool use_bitmap_plan(int32_t M, int32_t K, int64_t nnz, uint32_t flags);

// ---- bitmap plan (prune_bitmap.hip) -------------------------------------------
bool prune_bitmap_ok(int32_t M, int32_t K, int64_t nnz);
size_t prune_bitmap_ws_bytes(int32_t M, int32_t K, int64_t nnz);
snack_status prune_bitmap(int32_t* row, int32_t* col, void* vals, snack_dtype dt, int32_t M,
                          int32_t K, int64_t nnz, int64_t n_drop, uint64_t seed, uint64_t step,
                          int64_t* dropped_lin, int64_t* grown_lin, void* ws, hipStream_t s);
// The bitmap plan followed by the plan's derived arrays built from the new
// support bitmap (needs M, K multiples of 32).  plan: initialised for
// (M, K, nnz) with its arena; it describes the new COO on success.
bool prune_bitmap_fused_ok(int32_t M, int32_t K, int64_t nnz);
// vals_t (nullable) receives the new values in the new column order; rw:
// the plan's result words (internal.h).
struct result_words;
snack_status prune_bitmap_prepared(snack_plan* plan, int32_t* row, int32_t* col, void* vals,
                                   void* vals_t, snack_dtype dt, int64_t n_drop, uint64_t seed,
                                   uint64_t step, int64_t* dropped_lin, int64_t* grown_lin,
                                   void* ws, result_words& rw, hipStream_t s);

}  // namespace snk
