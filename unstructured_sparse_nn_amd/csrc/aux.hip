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

// Batch 1, bf16, K <= 4096 and a multiple of 8 (16-byte aligned rows): each
// wave takes two rows; lane l holds x[512 j + 8 l .. +7] for every j in
// registers, and the chunks of X and of both rows are requested together
// (16 KB of W per wave, the whole weight in flight over the GPU), so the
// product is one round trip of a non-temporal weight stream.
typedef uint32_t dn_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t dn_u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 dn_bf2 __attribute__((ext_vector_type(2)));
constexpr int G1_NC = 8;  // 512-wide chunks: K <= 4096

// The bf16 halves of w (elements 2e, 2e+1 of a chunk) whose mask byte is 0
// cleared; mm holds the chunk's 8 mask bytes.
__device__ __forceinline__ uint32_t mask_pair(uint32_t w, dn_u32x2 mm, int e) {
  const uint32_t mb = ((e < 2 ? mm.x : mm.y) >> (16 * (e & 1))) & 0xFFFFu;
  const uint32_t keep = ((mb & 0xFFu) ? 0x0000FFFFu : 0u) | ((mb >> 8) ? 0xFFFF0000u : 0u);
  return w & keep;
}

template <bool MASK>
__global__ __launch_bounds__(256) void k_dense_gemv1(const bf16* __restrict__ W,
                                                     const uint8_t* __restrict__ mask, int32_t M,
                                                     int32_t K, const bf16* __restrict__ X,
                                                     bf16* __restrict__ Y) {
  const int wv = threadIdx.x / SNK_WAVE, l = lane_id();
  const int32_t r0 = ((int32_t)blockIdx.x * 4 + wv) * 2;
  if (r0 >= M) return;
  const int32_t r1 = min(r0 + 1, M - 1);  // a missing second row repeats the first, unstored
  const dn_u32x4 z4 = {0u, 0u, 0u, 0u};
  const dn_u32x2 z2 = {0u, 0u};
  dn_u32x4 x[G1_NC], w0[G1_NC], w1[G1_NC];
  dn_u32x2 m0[G1_NC], m1[G1_NC];
#pragma unroll
  for (int j = 0; j < G1_NC; ++j) {
    const int32_t k = 512 * j + 8 * l;
    const bool ok = k < K;
    x[j] = ok ? *reinterpret_cast<const dn_u32x4*>(X + k) : z4;
    w0[j] = ok ? __builtin_nontemporal_load(
                     reinterpret_cast<const dn_u32x4*>(W + (int64_t)r0 * K + k))
               : z4;
    w1[j] = ok ? __builtin_nontemporal_load(
                     reinterpret_cast<const dn_u32x4*>(W + (int64_t)r1 * K + k))
               : z4;
    if (MASK) {
      m0[j] = ok ? __builtin_nontemporal_load(
                       reinterpret_cast<const dn_u32x2*>(mask + (int64_t)r0 * K + k))
                 : z2;
      m1[j] = ok ? __builtin_nontemporal_load(
                       reinterpret_cast<const dn_u32x2*>(mask + (int64_t)r1 * K + k))
                 : z2;
    }
  }
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int j = 0; j < G1_NC; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // vector elements are copied out first: a bit cast of the element
      // expression itself read element 0
      uint32_t p0 = w0[j][e], p1 = w1[j][e];
      const uint32_t xe = x[j][e];
      if (MASK) {
        p0 = mask_pair(p0, m0[j], e);
        p1 = mask_pair(p1, m1[j], e);
      }
      const dn_bf2 xv = __builtin_bit_cast(dn_bf2, xe);
      a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(dn_bf2, p0), xv, a0, false);
      a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(dn_bf2, p1), xv, a1, false);
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    a0 += __shfl_xor(a0, off, SNK_WAVE);
    a1 += __shfl_xor(a1, off, SNK_WAVE);
  }
  if (l == 0) {
    Y[r0] = f32_to_bf16(a0);
    if (r0 + 1 < M) Y[r0 + 1] = f32_to_bf16(a1);
  }
}

// bf16 batches of 16 or more on the matrix cores with 16-row output tiles
// (twice the workgroups of 32-row tiles, so that a 4096-row layer fills the
// 256 CUs): each workgroup owns 16 rows x 32 batch columns, its 8 waves
// split K, each step of 32 k is one v_mfma_f32_16x16x32_bf16 per 16 batch
// columns (lane l: row / column l mod 16, k 8 (l / 16) .. +7; the result's
// lane l holds column l mod 16, rows 4 (l / 16) .. +3), and the partial
// tiles are summed in LDS.
typedef __bf16 dn_bf8 __attribute__((ext_vector_type(8)));
typedef float dn_f4 __attribute__((ext_vector_type(4)));
constexpr int D16_WAVES = 8;
constexpr int D16_UNROLL = 4;

// 8 consecutive bf16 p[base + k .. +7] (0 past K or outside the mask).
template <bool MASK>
__device__ __forceinline__ dn_bf8 d16_load(const bf16* __restrict__ p,
                                           const uint8_t* __restrict__ m, int64_t base,
                                           int64_t k, int32_t K, bool ok, bool aligned) {
  uint32_t v[4] = {0u, 0u, 0u, 0u};
  if (ok) {
    if (aligned && k + 8 <= K) {
      const uint4 w = *reinterpret_cast<const uint4*>(p + base + k);
      v[0] = w.x;
      v[1] = w.y;
      v[2] = w.z;
      v[3] = w.w;
      if (MASK) {
        const uint2 mm = *reinterpret_cast<const uint2*>(m + base + k);
        const dn_u32x2 m2 = {mm.x, mm.y};
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = mask_pair(v[e], m2, e);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool in = k + e < K && (!MASK || m[base + k + e]);
        const uint32_t h = in ? (uint32_t)p[base + k + e] : 0u;
        v[e / 2] |= h << (16 * (e & 1));
      }
    }
  }
  return __builtin_bit_cast(dn_bf8, v);
}

template <bool MASK>
__global__ __launch_bounds__(64 * D16_WAVES) void k_dense_mfma16(
    const bf16* __restrict__ W, const uint8_t* __restrict__ mask, int32_t M, int32_t K,
    const bf16* __restrict__ X, int32_t B, bf16* __restrict__ Y, int32_t vec_ok) {
  __shared__ float part[D16_WAVES][2][4][64];
  const int wv = threadIdx.x / SNK_WAVE, l = lane_id();
  const int32_t r0 = blockIdx.x * 16, b0 = blockIdx.y * 32;
  const int32_t i = l & 15, q = l >> 4;
  const int32_t r = r0 + i, bA = b0 + i, bB = b0 + 16 + i;
  const bool r_ok = r < M, a_ok = bA < B, b_ok = bB < B;
  const int64_t wbase = (int64_t)r * K, xa = (int64_t)bA * K, xb = (int64_t)bB * K;
  const bool aligned = vec_ok && (K % 8) == 0;
  const int32_t groups = (K + 31) / 32;  // 32-wide k groups
  const int32_t per = (groups + D16_WAVES - 1) / D16_WAVES;
  const int32_t g0 = wv * per, g1 = min(groups, g0 + per);
  dn_f4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int32_t g = g0; g < g1; g += D16_UNROLL) {
    dn_bf8 a[D16_UNROLL], xa8[D16_UNROLL], xb8[D16_UNROLL];
#pragma unroll
    for (int u = 0; u < D16_UNROLL; ++u) {
      const int64_t k = (int64_t)(g + u) * 32 + 8 * q;
      const bool ok = g + u < g1;
      a[u] = d16_load<MASK>(W, mask, wbase, k, K, r_ok && ok, aligned);
      xa8[u] = d16_load<false>(X, nullptr, xa, k, K, a_ok && ok, aligned);
      xb8[u] = d16_load<false>(X, nullptr, xb, k, K, b_ok && ok, aligned);
    }
#pragma unroll
    for (int u = 0; u < D16_UNROLL; ++u) {
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], xa8[u], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], xb8[u], acc1, 0, 0, 0);
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    part[wv][0][v][l] = acc0[v];
    part[wv][1][v][l] = acc1[v];
  }
  __syncthreads();
  // 16 x 32 results, one per thread: row ri, batch column bj
  const int e = threadIdx.x;
  const int ri = e & 15, bj = e >> 4;
  const int half = bj >> 4, col = bj & 15;
  const int lane = col + 16 * (ri >> 2), v = ri & 3;
  float sum = 0.f;
#pragma unroll
  for (int w2 = 0; w2 < D16_WAVES; ++w2) sum += part[w2][half][v][lane];
  const int32_t rr = r0 + ri, bo = b0 + bj;
  if (rr < M && bo < B) Y[(int64_t)bo * M + rr] = f32_to_bf16(sum);
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
  const bool al16 = (uintptr_t)W % 16 == 0 && (uintptr_t)X % 16 == 0 && (uintptr_t)mask % 8 == 0;
  if (dt == SNACK_BF16 && B == 1 && al16 && K % 8 == 0 && K <= 512 * G1_NC) {
    const dim3 grid((unsigned)cdiv(M, 8));
    if (mask)
      hipLaunchKernelGGL(k_dense_gemv1<true>, grid, dim3(256), 0, s, (const bf16*)W, mask, M, K,
                         (const bf16*)X, (bf16*)Y);
    else
      hipLaunchKernelGGL(k_dense_gemv1<false>, grid, dim3(256), 0, s, (const bf16*)W, mask, M, K,
                         (const bf16*)X, (bf16*)Y);
    return hipGetLastError();
  }
  if (dt == SNACK_BF16 && B >= 16) {
    const dim3 grid((unsigned)cdiv(M, 16), (unsigned)cdiv(B, 32));
    const int32_t vec_ok = al16 ? 1 : 0;
    if (mask)
      hipLaunchKernelGGL(k_dense_mfma16<true>, grid, dim3(64 * D16_WAVES), 0, s, (const bf16*)W,
                         mask, M, K, (const bf16*)X, B, (bf16*)Y, vec_ok);
    else
      hipLaunchKernelGGL(k_dense_mfma16<false>, grid, dim3(64 * D16_WAVES), 0, s, (const bf16*)W,
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
