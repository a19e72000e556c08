// common.h -- device helpers shared by the gfx950 kernels of the sparse layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <utility>

#define SNK_WAVE 64

namespace snk {

typedef uint16_t bf16;  // raw bfloat16 bits

// Accelerator complex dies of an MI355X; workgroup b of a launch runs on die
// b mod NUM_XCD, and each die has its own L2.
constexpr int NUM_XCD = 8;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(bf16 h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Round to nearest, ties to even (IEEE 754 roundTiesToEven on the 16
// dropped mantissa bits); NaN stays a quiet NaN.
__device__ __forceinline__ bf16 f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (bf16)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16)(u >> 16);
}

template <typename T> struct elem;
template <> struct elem<float> {
  __device__ __forceinline__ static float to_f(float x) { return x; }
  __device__ __forceinline__ static float from_f(float x) { return x; }
};
template <> struct elem<bf16> {
  __device__ __forceinline__ static float to_f(bf16 x) { return bf16_to_f32(x); }
  __device__ __forceinline__ static bf16 from_f(float x) { return f32_to_bf16(x); }
};

// Vector of N elements of T, naturally aligned (N*sizeof(T) bytes), used to
// move a contiguous chunk of a node-major activation row in one access.
template <typename T, int N> struct __attribute__((aligned(N * sizeof(T)))) vec {
  T v[N];
};

template <typename T, int N>
__device__ __forceinline__ void load_vec(const T* __restrict__ p, float (&out)[N]) {
  vec<T, N> r = *reinterpret_cast<const vec<T, N>*>(p);
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = elem<T>::to_f(r.v[i]);
}

template <typename T, int N>
__device__ __forceinline__ void store_vec(T* __restrict__ p, const float (&in)[N]) {
  vec<T, N> r;
#pragma unroll
  for (int i = 0; i < N; ++i) r.v[i] = elem<T>::from_f(in[i]);
  *reinterpret_cast<vec<T, N>*>(p) = r;
}

// acc + sum_c a[c] * b[c] in fp32; bf16 pairs go through v_dot2_f32_bf16
// (exact bf16 products summed into the fp32 accumulator).
template <typename T, int CH>
__device__ __forceinline__ float dot_acc(const vec<T, CH>& a, const vec<T, CH>& b, float acc) {
  if constexpr (sizeof(T) == 2 && CH >= 2) {
    typedef __bf16 __attribute__((ext_vector_type(2))) bf2;
#pragma unroll
    for (int c = 0; c < CH; c += 2) {
      const uint32_t pa = (uint32_t)a.v[c] | ((uint32_t)a.v[c + 1] << 16);
      const uint32_t pb = (uint32_t)b.v[c] | ((uint32_t)b.v[c + 1] << 16);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, pa),
                                            __builtin_bit_cast(bf2, pb), acc, false);
    }
    return acc;
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) acc = fmaf(elem<T>::to_f(a.v[c]), elem<T>::to_f(b.v[c]), acc);
    return acc;
  }
}

// ---------------------------------------------------------------- activations
// Elementwise nonlinearity applied to a finished fp32 output before it is
// rounded and stored (0 none, 1 ReLU, 2 exact GELU).
enum { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2 };  // the values of snack_act

// Exact GELU: z * Phi(z), Phi(z) = (1 + erf(z / sqrt 2)) / 2.
__device__ __forceinline__ float gelu_f32(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

__device__ __forceinline__ float apply_act(float x, int32_t act) {
  if (act == ACT_RELU) return x > 0.f ? x : 0.f;
  if (act == ACT_GELU) return gelu_f32(x);
  return x;
}

// ---------------------------------------------------------------- lanes
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// ---------------------------------------------------------------- scans
__device__ __forceinline__ int32_t wave_incl_scan_i32(int32_t x) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < SNK_WAVE; d <<= 1) {
    int32_t y = __shfl_up(x, d, SNK_WAVE);
    if (l >= d) x += y;
  }
  return x;
}

// Exclusive prefix of one value per thread across a block of NTHREADS
// threads (a multiple of 64); *total receives the block sum.  lds must hold
// NTHREADS/64 ints.  Contains barriers: call from all threads.
template <int NTHREADS>
__device__ __forceinline__ int32_t block_excl_scan_i32(int32_t x, int32_t* lds, int32_t* total) {
  const int w = threadIdx.x / SNK_WAVE;
  const int32_t inc = wave_incl_scan_i32(x);
  if (lane_id() == SNK_WAVE - 1) lds[w] = inc;
  __syncthreads();
  int32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NTHREADS / SNK_WAVE; ++i) {
    const int32_t t = lds[i];
    if (i < w) base += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + inc - x;
}

// Add 1 to h[d] (LDS histogram of 256 bins) for every active lane with
// valid set, aggregating equal digits across the wave first: 8 ballots find
// the lanes sharing this lane's digit, the lowest of them adds the count.
// Skewed digit distributions then cost one LDS atomic per distinct digit.
__device__ __forceinline__ void wave_hist_add(int32_t* h, uint32_t d, bool valid) {
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint64_t m = __ballot((d >> b) & 1u);
    peers &= ((d >> b) & 1u) ? m : ~m;
  }
  if (valid && __popcll(peers & lanemask_lt()) == 0) atomicAdd(&h[d], __popcll(peers));
}

}  // namespace snk

#define SNK_CHECK_LAUNCH()                                   \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return SNACK_E_HIP; \
  } while (0)
