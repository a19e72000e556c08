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
  h[i] = gelu_f32(z[i]);
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

// y <- act(y) in place, 8 elements per thread (one 16- or 32-byte access
// when aligned), the GELU step of a propagation after its product.
template <typename T>
__global__ __launch_bounds__(256) void k_act_inplace(T* __restrict__ y, int64_t n, int32_t act) {
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i0 >= n) return;
  if (i0 + 8 <= n && (uintptr_t)(y + i0) % (8 * sizeof(T)) == 0) {
    vec<T, 8> v = *reinterpret_cast<const vec<T, 8>*>(y + i0);
#pragma unroll
    for (int e = 0; e < 8; ++e) v.v[e] = elem<T>::from_f(apply_act(elem<T>::to_f(v.v[e]), act));
    *reinterpret_cast<vec<T, 8>*>(y + i0) = v;
  } else {
    for (int64_t i = i0; i < n && i < i0 + 8; ++i)
      y[i] = elem<T>::from_f(apply_act(elem<T>::to_f(y[i]), act));
  }
}

hipError_t launch_act_inplace(snack_dtype dt, void* y, int64_t n, int32_t act, hipStream_t s) {
  if (n <= 0 || act == ACT_NONE) return hipSuccess;
  const dim3 grid((unsigned)cdiv(cdiv(n, 8), 256));
  if (dt == SNACK_F32) hipLaunchKernelGGL(k_act_inplace<float>, grid, dim3(256), 0, s, (float*)y, n, act);
  else hipLaunchKernelGGL(k_act_inplace<bf16>, grid, dim3(256), 0, s, (bf16*)y, n, act);
  return hipGetLastError();
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
// Y[b, r] = sum_k W[r, k] * mask[r, k] * X[b, k] with dense row-major W and
// batch-major X, Y.  A streaming reference for small batches: each wave owns
// RW rows and every batch column of its tile (BT <= 32), so W and the mask
// are read once; each lane takes 8 consecutive k per 512-wide chunk (16-byte
// loads of W, prefetched one chunk ahead), the chunk of X is staged in LDS
// for the whole workgroup, and the per-lane partial sums are reduced across
// the wave at the end.
constexpr int DN_KC = 512;  // K chunk: 64 lanes x 8

template <typename T>
__device__ __forceinline__ void load8(const T* __restrict__ p, int64_t k, int32_t K, float (&v)[8]) {
  if (k + 8 <= K && ((uintptr_t)(p + k) % (8 * sizeof(T))) == 0) {
    const vec<T, 8> w = *reinterpret_cast<const vec<T, 8>*>(p + k);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = elem<T>::to_f(w.v[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = k + e < K ? elem<T>::to_f(p[k + e]) : 0.f;
  }
}

template <typename T, bool MASK, int RW, int BT, int NTH>
__global__ __launch_bounds__(NTH) void k_dense_fwd(const T* __restrict__ W,
                                                          const uint8_t* __restrict__ mask,
                                                          int32_t M, int32_t K,
                                                          const T* __restrict__ X, int32_t B,
                                                          T* __restrict__ Y) {
  __shared__ T xs[BT][DN_KC];
  const int tid = threadIdx.x, wv = tid / SNK_WAVE, l = lane_id();
  const int32_t r0 = (blockIdx.x * (NTH / SNK_WAVE) + wv) * RW;
  const int32_t b0 = blockIdx.y * BT;
  float acc[RW][BT];
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int j = 0; j < BT; ++j) acc[i][j] = 0.f;
  float wn[RW][8];  // the next chunk of this lane's W elements
  auto fetch = [&](int32_t kc) {
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int32_t r = r0 + i;
      const int64_t k = (int64_t)kc + l * 8;
      if (r < M) {
        load8<T>(W + (int64_t)r * K, k, K, wn[i]);
        if (MASK) {
          const uint8_t* mp = mask + (int64_t)r * K + k;
          uint64_t m8 = 0;
          if (k + 8 <= K && (uintptr_t)mp % 8 == 0) {
            m8 = *reinterpret_cast<const uint64_t*>(mp);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) m8 |= (k + e < K ? (uint64_t)mp[e] : 0ull) << (8 * e);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (((m8 >> (8 * e)) & 0xFFu) == 0) wn[i][e] = 0.f;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) wn[i][e] = 0.f;
      }
    }
  };
  fetch(0);
  for (int32_t kc = 0; kc < K; kc += DN_KC) {
    float wc[RW][8];
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) wc[i][e] = wn[i][e];
    __syncthreads();  // previous chunk's xs reads done
    for (int e = tid; e < BT * DN_KC; e += NTH) {
      const int j = e / DN_KC, kk = e % DN_KC;
      const int32_t bb = b0 + j, k = kc + kk;
      xs[j][kk] = (bb < B && k < K) ? X[(int64_t)bb * K + k] : (T)0;
    }
    if (kc + DN_KC < K) fetch(kc + DN_KC);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < BT; ++j) {
      const vec<T, 8> xv = *reinterpret_cast<const vec<T, 8>*>(&xs[j][l * 8]);
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = elem<T>::to_f(xv.v[e]);
#pragma unroll
      for (int i = 0; i < RW; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][j] = fmaf(wc[i][e], x[e], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int j = 0; j < BT; ++j)
      for (int off = 32; off > 0; off >>= 1) acc[i][j] += __shfl_xor(acc[i][j], off, SNK_WAVE);
  if (l == 0) {
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int32_t r = r0 + i;
#pragma unroll
      for (int j = 0; j < BT; ++j) {
        const int32_t bb = b0 + j;
        if (r < M && bb < B) Y[(int64_t)bb * M + r] = elem<T>::from_f(acc[i][j]);
      }
    }
  }
}

// bf16, batch >= 16: a 32-row x 32-batch output tile per workgroup on the
// matrix cores (v_mfma_f32_32x32x8bf16_1k: D[i][j] += sum_k A[i][k] B[k][j]
// with A = 32 rows of W, B[k][j] = X[b0+j][k]).  In an 8-wide step lane l
// supplies A[l%32][4q..4q+3] and B[4q..4q+3][l%32] (q = l/32) and receives
// rows 8(v/4) + 4q + v%4 of column l%32 in its 16 results.  Which k feeds
// which step slot is free as long as A and B agree, so each lane loads 8
// consecutive k (16 bytes of W and of X) and feeds them to two steps.  The
// K axis is split over the DM_WAVES waves of the workgroup; the partial
// tiles are summed in LDS.
constexpr int DM_WAVES = 8;
constexpr int DM_UNROLL = 8;  // 16-wide k groups per iteration

typedef short dm_short4 __attribute__((ext_vector_type(4)));
typedef float dm_float16 __attribute__((ext_vector_type(16)));

// 8 consecutive bf16 p[base + k .. +7] (0 past K or outside the mask) as two
// MFMA fragments.
template <bool MASK>
__device__ __forceinline__ void dm_load8(const bf16* __restrict__ p, const uint8_t* __restrict__ m,
                                         int64_t base, int64_t k, int32_t K, bool ok, bool aligned,
                                         dm_short4& lo, dm_short4& hi) {
  lo = dm_short4{0, 0, 0, 0};
  hi = dm_short4{0, 0, 0, 0};
  if (!ok) return;
  short v[8];
  if (aligned && k + 8 <= K) {
    const uint4 w = *reinterpret_cast<const uint4*>(p + base + k);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = (short)(ws[e] & 0xFFFFu);
      v[2 * e + 1] = (short)(ws[e] >> 16);
    }
    if (MASK) {
      const uint2 mm = *reinterpret_cast<const uint2*>(m + base + k);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((((e < 4 ? mm.x : mm.y) >> (8 * (e & 3))) & 0xFFu) == 0) v[e] = 0;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool in = k + e < K && (!MASK || m[base + k + e]);
      v[e] = in ? (short)p[base + k + e] : (short)0;
    }
  }
  lo = dm_short4{v[0], v[1], v[2], v[3]};
  hi = dm_short4{v[4], v[5], v[6], v[7]};
}

template <bool MASK>
__global__ __launch_bounds__(64 * DM_WAVES) void k_dense_mfma(const bf16* __restrict__ W,
                                                              const uint8_t* __restrict__ mask,
                                                              int32_t M, int32_t K,
                                                              const bf16* __restrict__ X,
                                                              int32_t B, bf16* __restrict__ Y,
                                                              int32_t vec_ok) {
  __shared__ float part[DM_WAVES][16][64];
  const int wv = threadIdx.x / SNK_WAVE, l = lane_id();
  const int32_t r0 = blockIdx.x * 32, b0 = blockIdx.y * 32;
  const int32_t i = l & 31, q = l >> 5;
  const int32_t r = r0 + i, b = b0 + i;
  const bool r_ok = r < M, b_ok = b < B;
  const int64_t wbase = (int64_t)r * K, xbase = (int64_t)b * K;
  const bool aligned = vec_ok && (K % 8) == 0;
  // this wave's share of the K axis, in 16-wide groups
  const int32_t groups = (K + 15) / 16;
  const int32_t per = (groups + DM_WAVES - 1) / DM_WAVES;
  const int32_t g0 = wv * per, g1 = min(groups, g0 + per);
  dm_float16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  for (int32_t g = g0; g < g1; g += DM_UNROLL) {
    dm_short4 alo[DM_UNROLL], ahi[DM_UNROLL], blo[DM_UNROLL], bhi[DM_UNROLL];
#pragma unroll
    for (int u = 0; u < DM_UNROLL; ++u) {
      const int64_t k = (int64_t)(g + u) * 16 + 8 * q;
      const bool ok = g + u < g1;
      dm_load8<MASK>(W, mask, wbase, k, K, r_ok && ok, aligned, alo[u], ahi[u]);
      dm_load8<false>(X, nullptr, xbase, k, K, b_ok && ok, aligned, blo[u], bhi[u]);
    }
#pragma unroll
    for (int u = 0; u < DM_UNROLL; ++u) {
      acc = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(alo[u], blo[u], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(ahi[u], bhi[u], acc, 0, 0, 0);
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) part[wv][v][l] = acc[v];
  __syncthreads();
  // 16 x 64 results; the workgroup's 512 threads take two each
  for (int e = threadIdx.x; e < 16 * 64; e += 64 * DM_WAVES) {
    const int v = e / 64, ll = e % 64;
    float sum = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < DM_WAVES; ++w2) sum += part[w2][v][ll];
    const int32_t rr = r0 + 8 * (v / 4) + 4 * (ll >> 5) + (v % 4);
    const int32_t bo = b0 + (ll & 31);
    if (rr < M && bo < B) Y[(int64_t)bo * M + rr] = f32_to_bf16(sum);
  }
}

// Small batches (B <= 8) as a weight stream: each wave owns RW rows and the
// whole batch; per 512-wide step each lane takes 8 consecutive k (16 bytes
// of bf16 W, 32 of fp32), and U steps' loads of W, of the mask and of X (read
// from the caches: every wave reads the same X) are all issued before any of
// them is used (at batch 1, 8 KB of W per wave, 16 MB over the GPU, in
// flight at once).  No LDS, no barrier; the lane
// partial sums are reduced across the wave at the end.
template <typename T, bool MASK, int RW, int BT, int U>
__global__ __launch_bounds__(256) void k_dense_stream(const T* __restrict__ W,
                                                      const uint8_t* __restrict__ mask, int32_t M,
                                                      int32_t K, const T* __restrict__ X,
                                                      int32_t B, T* __restrict__ Y,
                                                      int32_t vec_ok) {
  const int wv = threadIdx.x / SNK_WAVE, l = lane_id();
  const int32_t r0 = (int32_t)(blockIdx.x * 4 + wv) * RW;
  if (r0 >= M) return;
  const bool aligned = vec_ok && (K % 8) == 0;
  float acc[RW][BT];
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int j = 0; j < BT; ++j) acc[i][j] = 0.f;
  for (int32_t kc = 0; kc < K; kc += U * DN_KC) {
    vec<T, 8> w[U][RW], x[U][BT];
    uint2 m[U][RW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (int64_t)kc + u * DN_KC + l * 8;
      const bool full = aligned && k + 8 <= K;
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const int32_t r = min(r0 + i, M - 1);  // rows past M add into acc rows never stored
        const T* p = W + (int64_t)r * K;
        if (full) {
          w[u][i] = *reinterpret_cast<const vec<T, 8>*>(p + k);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) w[u][i].v[e] = k + e < K ? p[k + e] : (T)0;
        }
        if (MASK) {
          const uint8_t* mp = mask + (int64_t)r * K;
          if (full) {
            m[u][i] = *reinterpret_cast<const uint2*>(mp + k);
          } else {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t b = k + e < K ? mp[k + e] : 0u;
              if (e < 4) lo |= b << (8 * e);
              else hi |= b << (8 * (e - 4));
            }
            m[u][i] = make_uint2(lo, hi);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < BT; ++j) {
        const int32_t b = min(j, B - 1);  // batch columns past B are never stored
        const T* p = X + (int64_t)b * K;
        if (full) {
          x[u][j] = *reinterpret_cast<const vec<T, 8>*>(p + k);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[u][j].v[e] = k + e < K ? p[k + e] : (T)0;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        float wf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          wf[e] = elem<T>::to_f(w[u][i].v[e]);
          if (MASK && (((e < 4 ? m[u][i].x : m[u][i].y) >> (8 * (e & 3))) & 0xFFu) == 0)
            wf[e] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < BT; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc[i][j] = fmaf(wf[e], elem<T>::to_f(x[u][j].v[e]), acc[i][j]);
      }
  }
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int j = 0; j < BT; ++j)
      for (int off = 32; off > 0; off >>= 1) acc[i][j] += __shfl_xor(acc[i][j], off, SNK_WAVE);
  if (l == 0) {
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
      for (int j = 0; j < BT; ++j)
        if (r0 + i < M && j < B) Y[(int64_t)j * M + r0 + i] = elem<T>::from_f(acc[i][j]);
  }
}

// Batches up to 8 take the weight stream; wider ones stage chunks of X in
// LDS, with rows per workgroup growing with the batch tile, so that the
// staged chunk is shared by enough rows (16 rows for 32 batch columns).
template <typename T, bool MASK>
static void launch_dense(const T* W, const uint8_t* mask, int32_t M, int32_t K, const T* X,
                         int32_t B, T* Y, hipStream_t s) {
  constexpr int w16 = 16;  // waves per workgroup
  const int32_t vec_ok = ((uintptr_t)W % 32 == 0 && (uintptr_t)X % 32 == 0 &&
                          (uintptr_t)mask % 8 == 0) ? 1 : 0;
  // two rows per wave, four waves per workgroup (measured at 4096^2 bf16,
  // batch 1: 13.6 us, against 16.5 us with one row of 8 steps per wave); the
  // steps in flight shrink as the batch (the X chunks held per step) grows
  const dim3 g2((unsigned)cdiv(M, 4 * 2));
  if (B <= 1) {
    hipLaunchKernelGGL((k_dense_stream<T, MASK, 2, 1, 4>), g2, dim3(256), 0, s, W, mask, M, K, X,
                       B, Y, vec_ok);
  } else if (B <= 2) {
    hipLaunchKernelGGL((k_dense_stream<T, MASK, 2, 2, 4>), g2, dim3(256), 0, s, W, mask, M, K, X,
                       B, Y, vec_ok);
  } else if (B <= 4) {
    hipLaunchKernelGGL((k_dense_stream<T, MASK, 2, 4, 2>), g2, dim3(256), 0, s, W, mask, M, K, X,
                       B, Y, vec_ok);
  } else if (B <= 8) {
    hipLaunchKernelGGL((k_dense_stream<T, MASK, 2, 8, 2>), g2, dim3(256), 0, s, W, mask, M, K, X,
                       B, Y, vec_ok);
  } else {
    hipLaunchKernelGGL((k_dense_fwd<T, MASK, 1, 32, 64 * w16>),
                       dim3((unsigned)cdiv(M, w16), (unsigned)cdiv(B, 32)), dim3(64 * w16), 0, s,
                       W, mask, M, K, X, B, Y);
  }
}

hipError_t launch_dense_fwd(const void* W, const uint8_t* mask, snack_dtype dt, int32_t M,
                            int32_t K, const void* X, int32_t B, void* Y, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (dt == SNACK_BF16 && B >= 16) {
    const dim3 grid((unsigned)cdiv(M, 32), (unsigned)cdiv(B, 32));
    const int32_t vec_ok = ((uintptr_t)W % 16 == 0 && (uintptr_t)X % 16 == 0 &&
                            (uintptr_t)mask % 8 == 0) ? 1 : 0;
    if (mask)
      hipLaunchKernelGGL(k_dense_mfma<true>, grid, dim3(64 * DM_WAVES), 0, s, (const bf16*)W,
                         mask, M, K, (const bf16*)X, B, (bf16*)Y, vec_ok);
    else
      hipLaunchKernelGGL(k_dense_mfma<false>, grid, dim3(64 * DM_WAVES), 0, s, (const bf16*)W,
                         mask, M, K, (const bf16*)X, B, (bf16*)Y, vec_ok);
    return hipGetLastError();
  }
  if (dt == SNACK_F32) {
    if (mask) launch_dense<float, true>((const float*)W, mask, M, K, (const float*)X, B, (float*)Y, s);
    else launch_dense<float, false>((const float*)W, mask, M, K, (const float*)X, B, (float*)Y, s);
  } else {
    if (mask) launch_dense<bf16, true>((const bf16*)W, mask, M, K, (const bf16*)X, B, (bf16*)Y, s);
    else launch_dense<bf16, false>((const bf16*)W, mask, M, K, (const bf16*)X, B, (bf16*)Y, s);
  }
  return hipGetLastError();
}

}  // namespace snk
