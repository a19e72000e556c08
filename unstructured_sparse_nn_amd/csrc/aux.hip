// aux.hip -- GELU between the two sparse layers of an MLP block, and the
// dense / dense+mask baselines the SNACK abstract compares against (gfx950).
#include "common.h"
#include "internal.h"

namespace snk {

// Exact GELU: h = z * Phi(z), Phi(z) = (1 + erf(z / sqrt 2)) / 2.
__global__ __launch_bounds__(256) void k_gelu_fwd(const float* __restrict__ z,
                                                  float* __restrict__ h, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float x = z[i];
  h[i] = 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

// dz = dh * (Phi(z) + z * phi(z)), phi(z) = exp(-z^2/2) / sqrt(2 pi).
__global__ __launch_bounds__(256) void k_gelu_bwd(const float* __restrict__ z,
                                                  const float* __restrict__ dh,
                                                  float* __restrict__ dz, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float x = z[i];
  float cdf = 0.5f * (1.0f + erff(x * 0.70710678118654752f));
  float pdf = 0.39894228040143267794f * expf(-0.5f * x * x);
  dz[i] = dh[i] * (cdf + x * pdf);
}

hipError_t launch_gelu_fwd(const float* z, float* h, int64_t n, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(k_gelu_fwd, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, z, h, n);
  return hipGetLastError();
}

hipError_t launch_gelu_bwd(const float* z, const float* dh, float* dz, int64_t n,
                           hipStream_t s) {
  if (n > 0)
    hipLaunchKernelGGL(k_gelu_bwd, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, z, dh, dz, n);
  return hipGetLastError();
}

// ------------------------------------------------------------ dense baseline
// Y[b, r] = sum_k W[r, k] * mask[r, k] * X[b, k] with dense row-major W.
// Streaming layout for small batches: a workgroup owns DN_ROWS rows and
// DN_BT batch columns; the K axis is walked in chunks of 512 (8 elements per
// lane); the chunk of X is staged in LDS once per workgroup and reused by all
// its rows; W (and the mask) stream from HBM with 8-element vector loads.
constexpr int DN_THREADS = 256;
constexpr int DN_RPW = 4;                 // rows per wave
constexpr int DN_ROWS = 4 * DN_RPW;       // rows per workgroup
constexpr int DN_BT = 8;                  // batch columns per workgroup
constexpr int DN_KC = 512;                // K chunk

template <typename T, bool MASK>
__global__ __launch_bounds__(DN_THREADS) void k_dense_fwd(const T* __restrict__ W,
                                                          const uint8_t* __restrict__ mask,
                                                          int32_t M, int32_t K,
                                                          const T* __restrict__ X, int32_t B,
                                                          T* __restrict__ Y) {
  __shared__ float xs[DN_BT][DN_KC];
  const int tid = threadIdx.x, w = tid / SNK_WAVE, l = lane_id();
  const int32_t r0 = blockIdx.x * DN_ROWS + w * DN_RPW;
  const int32_t b0 = blockIdx.y * DN_BT;
  float acc[DN_RPW][DN_BT];
#pragma unroll
  for (int i = 0; i < DN_RPW; ++i)
#pragma unroll
    for (int j = 0; j < DN_BT; ++j) acc[i][j] = 0.f;

  for (int32_t kc = 0; kc < K; kc += DN_KC) {
    for (int e = tid; e < DN_BT * DN_KC; e += DN_THREADS) {
      int j = e / DN_KC, kk = e % DN_KC;
      int32_t b = b0 + j, k = kc + kk;
      xs[j][kk] = (b < B && k < K) ? elem<T>::to_f(X[(int64_t)b * K + k]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < DN_RPW; ++i) {
      const int32_t r = r0 + i;
      if (r >= M) break;
      float wv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int32_t k = kc + l * 8 + e;
        float x = 0.f;
        if (k < K) {
          x = elem<T>::to_f(W[(int64_t)r * K + k]);
          if (MASK && !mask[(int64_t)r * K + k]) x = 0.f;
        }
        wv[e] = x;
      }
#pragma unroll
      for (int j = 0; j < DN_BT; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][j] = fmaf(wv[e], xs[j][l * 8 + e], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < DN_RPW; ++i)
#pragma unroll
    for (int j = 0; j < DN_BT; ++j)
      for (int off = 32; off > 0; off >>= 1) acc[i][j] += __shfl_xor(acc[i][j], off, SNK_WAVE);
  if (l == 0) {
#pragma unroll
    for (int i = 0; i < DN_RPW; ++i) {
      const int32_t r = r0 + i;
#pragma unroll
      for (int j = 0; j < DN_BT; ++j) {
        const int32_t b = b0 + j;
        if (r < M && b < B) Y[(int64_t)b * M + r] = elem<T>::from_f(acc[i][j]);
      }
    }
  }
}

hipError_t launch_dense_fwd(const void* W, const uint8_t* mask, snack_dtype dt, int32_t M,
                            int32_t K, const void* X, int32_t B, void* Y, hipStream_t s) {
  if (B == 0) return hipSuccess;
  dim3 grid((unsigned)cdiv(M, DN_ROWS), (unsigned)cdiv(B, DN_BT));
  if (dt == SNACK_F32) {
    if (mask)
      hipLaunchKernelGGL((k_dense_fwd<float, true>), grid, dim3(DN_THREADS), 0, s,
                         (const float*)W, mask, M, K, (const float*)X, B, (float*)Y);
    else
      hipLaunchKernelGGL((k_dense_fwd<float, false>), grid, dim3(DN_THREADS), 0, s,
                         (const float*)W, mask, M, K, (const float*)X, B, (float*)Y);
  } else {
    if (mask)
      hipLaunchKernelGGL((k_dense_fwd<bf16, true>), grid, dim3(DN_THREADS), 0, s,
                         (const bf16*)W, mask, M, K, (const bf16*)X, B, (bf16*)Y);
    else
      hipLaunchKernelGGL((k_dense_fwd<bf16, false>), grid, dim3(DN_THREADS), 0, s,
                         (const bf16*)W, mask, M, K, (const bf16*)X, B, (bf16*)Y);
  }
  return hipGetLastError();
}

}  // namespace snk
