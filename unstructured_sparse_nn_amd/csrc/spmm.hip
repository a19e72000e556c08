// spmm.hip -- sparse x dense products of the truly sparse layer (gfx950).
//
// One kernel serves both products the layer needs ("Beyond Masked Sparsity:
// SNACK Enables Truly Sparse Neural Networks on GPU", Abstract: compute only
// the nonzero connections, forward and backward):
//   forward   Y  = X W^T  over the row view    (segments = rows,    idx = col)
//   backward  dX = dY W   over the column view (segments = columns, idx = row,
//                                               values through perm)
// It computes, for every segment s and batch column b,
//     out[b, s] = sum_{k in segment s} v[k] * in[b, idx[k]].
//
// Work split (answers "Two Lotteries", paragraphs on gathers and on who does
// the work):
//   * one 256-thread workgroup per load-balanced tile of < 2T merge-path
//     items (segment ends + entries), so a long row costs the same per tile
//     as many short ones;
//   * inside a tile, G lanes form an item group that owns CH consecutive batch
//     columns each (one 4-16 byte access per entry for node-major
//     activations); the 256/G groups cut the tile's merge path into equal
//     runs and walk them serially, keeping the running sum in registers and
//     writing each segment they finish;
//   * entries of a run are fetched RC at a time: indices and values first,
//     then all RC activation gathers, so each wave keeps many loads in
//     flight;
//   * a segment cut by a run boundary is finished deterministically: partial
//     sums of the groups before it are added in group order through LDS, and
//     a segment cut by a tile boundary (only segments with >= T entries) goes
//     through per-tile carry slots summed in tile order by k_fixup.
// No floating-point atomics: results are bitwise reproducible.
#include "common.h"
#include "internal.h"

namespace snk {

constexpr int MP_THREADS = 256;
constexpr int MP_TMAX = 2048;              // largest tile size (items)
constexpr int MP_SEG_LDS = 2 * MP_TMAX;    // a tile holds < 2T segment ends
constexpr int MP_RC = 8;                   // entries fetched per step

template <typename T, int CH, bool NODE>
__device__ __forceinline__ void gather_in(const T* __restrict__ X, int32_t f, int32_t b0,
                                          int32_t B, int32_t F, float (&out)[CH]) {
  if constexpr (NODE) {
    load_vec<T, CH>(X + (int64_t)f * B + b0, out);
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) out[c] = elem<T>::to_f(X[(int64_t)(b0 + c) * F + f]);
  }
}

template <typename T, int CH, bool NODE>
__device__ __forceinline__ void store_out(T* __restrict__ Y, int32_t s, int32_t b0, int32_t B,
                                          int32_t S, const float (&v)[CH]) {
  if constexpr (NODE) {
    store_vec<T, CH>(Y + (int64_t)s * B + b0, v);
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) Y[(int64_t)(b0 + c) * S + s] = elem<T>::from_f(v[c]);
  }
}

// Merge-path point of local diagonal d inside a tile: the number x of
// segment ends consumed (end x' is consumed before entry j iff
// end[x'] <= j).
__device__ __forceinline__ int tile_search(const int32_t* s_end, int d, int nseg, int nz,
                                           int32_t zb) {
  int lo = max(0, d - nz), hi = min(d, nseg);
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (s_end[mid] <= zb + (d - mid - 1)) lo = mid + 1; else hi = mid;
  }
  return lo;
}

template <typename T, int CH, bool NODE, bool PERM>
__global__ __launch_bounds__(MP_THREADS) void k_seg_spmm(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm, const T* __restrict__ vals,
    const int32_t* __restrict__ part_seg, const int32_t* __restrict__ part_nz,
    const T* __restrict__ X, T* __restrict__ Y, float* __restrict__ carry, int32_t S, int32_t F,
    int32_t B, int32_t P, int32_t g_log2) {
  __shared__ int32_t s_end[MP_SEG_LDS];
  __shared__ int32_t s_gx[MP_THREADS + 1];
  __shared__ int32_t s_gy[MP_THREADS + 1];
  __shared__ int32_t s_cseg[MP_THREADS];
  __shared__ float s_cval[MP_THREADS * CH];

  const int G = 1 << g_log2;
  const int NT = MP_THREADS >> g_log2;
  const int tid = threadIdx.x;
  const int grp = tid >> g_log2;
  const int gl = tid & (G - 1);
  const int p = blockIdx.x;
  const int32_t b0 = (int32_t)blockIdx.y * (G * CH) + gl * CH;
  const bool bvalid = b0 < B;

  const int32_t sb = part_seg[p], zb = part_nz[p];
  const int32_t se = part_seg[p + 1], ze = part_nz[p + 1];
  const int nseg = se - sb;
  const int nz = ze - zb;
  const int items = nseg + nz;
  const int32_t seg0_start = ptr[sb];

  for (int i = tid; i < nseg; i += MP_THREADS) s_end[i] = ptr[sb + 1 + i];
  __syncthreads();

  const int R = (items + NT - 1) / NT;
  if (gl == 0) {
    int d = min(grp * R, items);
    int x = tile_search(s_end, d, nseg, nz, zb);
    s_gx[grp] = x;
    s_gy[grp] = d - x;
  }
  if (tid == 0) {
    s_gx[NT] = nseg;
    s_gy[NT] = nz;
  }
  __syncthreads();
  const int x0 = s_gx[grp], y0 = s_gy[grp];
  const int x1 = s_gx[grp + 1], y1 = s_gy[grp + 1];
  const int32_t x0_start = (x0 == 0) ? seg0_start : s_end[min(x0, MP_SEG_LDS) - 1];
  const bool mid_start = (zb + y0) > x0_start;
  const bool tile_carry_in = zb > seg0_start;

  float acc[CH], pend[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) acc[c] = pend[c] = 0.f;
  bool has_pend = false, first_emit = true;
  int x = x0;

  auto emit = [&](int xx) {
    if (first_emit && mid_start) {
#pragma unroll
      for (int c = 0; c < CH; ++c) pend[c] = acc[c];
      has_pend = true;
    } else if (bvalid) {
      store_out<T, CH, NODE>(Y, sb + xx, b0, B, S, acc);
    }
    first_emit = false;
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = 0.f;
  };

  for (int y = y0; y < y1; y += MP_RC) {
    const int n = min(MP_RC, y1 - y);
    int32_t ci[MP_RC];
    float cv[MP_RC];
    float xv[MP_RC][CH];
#pragma unroll
    for (int u = 0; u < MP_RC; ++u) {
      if (u < n) {
        int64_t k = (int64_t)zb + y + u;
        ci[u] = idx[k];
        cv[u] = elem<T>::to_f(PERM ? vals[perm[k]] : vals[k]);
      }
    }
#pragma unroll
    for (int u = 0; u < MP_RC; ++u) {
      if (u < n && bvalid) {
        gather_in<T, CH, NODE>(X, ci[u], b0, B, F, xv[u]);
      } else {
#pragma unroll
        for (int c = 0; c < CH; ++c) xv[u][c] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < MP_RC; ++u) {
      if (u < n) {
        const int32_t kg = zb + y + u;
        while (x < x1 && s_end[x] <= kg) emit(x++);
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] = fmaf(cv[u], xv[u][c], acc[c]);
      }
    }
  }
  while (x < x1) emit(x++);

  s_cseg[grp] = x1;  // written by every lane of the group (same value)
#pragma unroll
  for (int c = 0; c < CH; ++c) s_cval[tid * CH + c] = acc[c];
  __syncthreads();

  if (has_pend) {
    int t = grp - 1;
    while (t >= 0 && s_cseg[t] == x0) --t;
    float tot[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) tot[c] = 0.f;
    for (int u = t + 1; u < grp; ++u) {
#pragma unroll
      for (int c = 0; c < CH; ++c) tot[c] += s_cval[(u * G + gl) * CH + c];
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) tot[c] += pend[c];
    if (bvalid) {
      if (x0 == 0 && tile_carry_in) {
        float* dst = carry + ((int64_t)P + p) * B + b0;
#pragma unroll
        for (int c = 0; c < CH; ++c) dst[c] = tot[c];
      } else {
        store_out<T, CH, NODE>(Y, sb + x0, b0, B, S, tot);
      }
    }
  }

  if (grp == NT - 1 && bvalid) {
    const int32_t trail_start = (nseg == 0) ? seg0_start : s_end[nseg - 1];
    if (ze > max(zb, trail_start)) {
      int t = NT - 1;
      while (t >= 0 && s_cseg[t] == nseg) --t;
      float tot[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) tot[c] = 0.f;
      for (int u = t + 1; u < NT; ++u) {
#pragma unroll
        for (int c = 0; c < CH; ++c) tot[c] += s_cval[(u * G + gl) * CH + c];
      }
      float* dst = carry + (int64_t)p * B + b0;
#pragma unroll
      for (int c = 0; c < CH; ++c) dst[c] = tot[c];
    }
  }
}

// Segments cut by tile boundaries: out = sum of the carry-out slots of tiles
// first..last-1 (in tile order) + the final piece held by tile `last`.
template <typename T, bool NODE>
__global__ __launch_bounds__(256) void k_fixup(const int32_t* __restrict__ split, int32_t n_split,
                                               const float* __restrict__ carry, T* __restrict__ Y,
                                               int32_t S, int32_t B, int32_t P) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)n_split * B) return;
  int32_t j = (int32_t)(i / B), b = (int32_t)(i % B);
  int32_t s = split[3 * j], f = split[3 * j + 1], l = split[3 * j + 2];
  float tot = 0.f;
  for (int32_t q = f; q < l; ++q) tot += carry[(int64_t)q * B + b];
  tot += carry[((int64_t)P + l) * B + b];
  if (NODE) Y[(int64_t)s * B + b] = elem<T>::from_f(tot);
  else Y[(int64_t)b * S + s] = elem<T>::from_f(tot);
}

// dV[k] = sum_b dY[b, seg(k)] * X[b, idx[k]], walking the same tiles to learn
// each entry's segment without reading a per-entry row index.
template <typename T, int CH, bool NODE>
__global__ __launch_bounds__(MP_THREADS) void k_sddmm(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ part_seg, const int32_t* __restrict__ part_nz,
    const T* __restrict__ dY, const T* __restrict__ X, T* __restrict__ dV, int32_t S, int32_t F,
    int32_t B, int32_t g_log2) {
  __shared__ int32_t s_end[MP_SEG_LDS];
  __shared__ int32_t s_gx[MP_THREADS + 1];
  __shared__ int32_t s_gy[MP_THREADS + 1];

  const int G = 1 << g_log2;
  const int NT = MP_THREADS >> g_log2;
  const int tid = threadIdx.x;
  const int grp = tid >> g_log2;
  const int gl = tid & (G - 1);
  const int p = blockIdx.x;
  const int BW = G * CH;

  const int32_t sb = part_seg[p], zb = part_nz[p];
  const int32_t se = part_seg[p + 1], ze = part_nz[p + 1];
  const int nseg = se - sb;
  const int nz = ze - zb;
  const int items = nseg + nz;

  for (int i = tid; i < nseg; i += MP_THREADS) s_end[i] = ptr[sb + 1 + i];
  __syncthreads();
  const int R = (items + NT - 1) / NT;
  if (gl == 0) {
    int d = min(grp * R, items);
    int x = tile_search(s_end, d, nseg, nz, zb);
    s_gx[grp] = x;
    s_gy[grp] = d - x;
  }
  if (tid == 0) {
    s_gx[NT] = nseg;
    s_gy[NT] = nz;
  }
  __syncthreads();
  const int x1 = s_gx[grp + 1], y0 = s_gy[grp], y1 = s_gy[grp + 1];
  int x = s_gx[grp];

  for (int y = y0; y < y1; y += MP_RC) {
    const int n = min(MP_RC, y1 - y);
    int32_t ci[MP_RC], sg[MP_RC];
    float dot[MP_RC];
#pragma unroll
    for (int u = 0; u < MP_RC; ++u) {
      dot[u] = 0.f;
      ci[u] = 0;
      sg[u] = sb;
      if (u < n) {
        const int32_t kg = zb + y + u;
        ci[u] = idx[kg];
        while (x < x1 && s_end[x] <= kg) ++x;
        sg[u] = sb + x;
      }
    }
    for (int32_t bb = 0; bb < B; bb += BW) {
      const int32_t b0 = bb + gl * CH;
      if (b0 < B) {
#pragma unroll
        for (int u = 0; u < MP_RC; ++u) {
          if (u < n) {
            float xv[CH], gv[CH];
            gather_in<T, CH, NODE>(X, ci[u], b0, B, F, xv);
            gather_in<T, CH, NODE>(dY, sg[u], b0, B, S, gv);
#pragma unroll
            for (int c = 0; c < CH; ++c) dot[u] = fmaf(gv[c], xv[c], dot[u]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < MP_RC; ++u) {
      for (int off = 1; off < G; off <<= 1) dot[u] += __shfl_xor(dot[u], off, SNK_WAVE);
    }
    if (gl == 0) {
#pragma unroll
      for (int u = 0; u < MP_RC; ++u)
        if (u < n) dV[(int64_t)zb + y + u] = elem<T>::from_f(dot[u]);
    }
  }
}

template <typename T>
__global__ void k_fill_zero(T* __restrict__ p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = (T)0;
}

// ---------------------------------------------------------------- host side
struct lane_shape {
  int ch;      // batch columns per lane
  int g_log2;  // lanes per item group = 1 << g_log2
  int bw;      // batch columns per workgroup
};

static lane_shape pick_shape(snack_dtype dt, int32_t B) {
  const int chmax = dt == SNACK_BF16 ? 8 : 4;
  int ch = 1;
  while (ch < chmax && B % (ch * 2) == 0) ch *= 2;
  int want = (int)std::min<int64_t>(cdiv(B, ch), 32 / ch);
  int g_log2 = 0;
  while ((1 << g_log2) < want) ++g_log2;
  return {ch, g_log2, ch << g_log2};
}

template <typename T, int CH, bool NODE, bool PERM>
static void launch_t(const seg_view& v, const void* vals, const void* X, int32_t B, void* Y,
                     float* carry, int g_log2, int bw, hipStream_t s) {
  dim3 grid((unsigned)v.P, (unsigned)cdiv(B, bw));
  hipLaunchKernelGGL((k_seg_spmm<T, CH, NODE, PERM>), grid, dim3(MP_THREADS), 0, s, v.ptr,
                     v.idx, v.perm, (const T*)vals, v.part_seg, v.part_nz, (const T*)X, (T*)Y,
                     carry, v.S, v.F, B, v.P, g_log2);
  if (v.n_split > 0) {
    int64_t n = (int64_t)v.n_split * B;
    hipLaunchKernelGGL((k_fixup<T, NODE>), dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s,
                       v.split, v.n_split, carry, (T*)Y, v.S, B, v.P);
  }
}

template <typename T, int CH>
static void launch_ch(const seg_view& v, const void* vals, const void* X, snack_layout lay,
                      int32_t B, void* Y, float* carry, int g_log2, int bw, hipStream_t s) {
  const bool node = lay == SNACK_NODE_MAJOR;
  const bool perm = v.perm != nullptr;
  if (node && perm) launch_t<T, CH, true, true>(v, vals, X, B, Y, carry, g_log2, bw, s);
  else if (node) launch_t<T, CH, true, false>(v, vals, X, B, Y, carry, g_log2, bw, s);
  else if (perm) launch_t<T, CH, false, true>(v, vals, X, B, Y, carry, g_log2, bw, s);
  else launch_t<T, CH, false, false>(v, vals, X, B, Y, carry, g_log2, bw, s);
}

template <typename T>
static void launch_dt(const seg_view& v, const void* vals, const void* X, snack_layout lay,
                      int32_t B, void* Y, float* carry, const lane_shape& sh, hipStream_t s) {
  switch (sh.ch) {
    case 1: launch_ch<T, 1>(v, vals, X, lay, B, Y, carry, sh.g_log2, sh.bw, s); break;
    case 2: launch_ch<T, 2>(v, vals, X, lay, B, Y, carry, sh.g_log2, sh.bw, s); break;
    case 4: launch_ch<T, 4>(v, vals, X, lay, B, Y, carry, sh.g_log2, sh.bw, s); break;
    default:
      if constexpr (sizeof(T) == 2) launch_ch<T, 8>(v, vals, X, lay, B, Y, carry, sh.g_log2, sh.bw, s);
      break;
  }
}

snack_status launch_seg_spmm(const seg_view& v, const void* vals, snack_dtype dt, const void* X,
                             snack_layout lay, int32_t B, void* Y, float* carry, hipStream_t s) {
  if (B == 0 || v.S == 0) return SNACK_OK;
  lane_shape sh = pick_shape(dt, B);
  if (dt == SNACK_F32) launch_dt<float>(v, vals, X, lay, B, Y, carry, sh, s);
  else launch_dt<bf16>(v, vals, X, lay, B, Y, carry, sh, s);
  return hipGetLastError() == hipSuccess ? SNACK_OK : SNACK_E_HIP;
}

template <typename T, int CH>
static void launch_sddmm_ch(const seg_view& v, const void* dY, const void* X, snack_layout lay,
                            int32_t B, void* dV, int g_log2, hipStream_t s) {
  dim3 grid((unsigned)v.P);
  if (lay == SNACK_NODE_MAJOR)
    hipLaunchKernelGGL((k_sddmm<T, CH, true>), grid, dim3(MP_THREADS), 0, s, v.ptr, v.idx,
                       v.part_seg, v.part_nz, (const T*)dY, (const T*)X, (T*)dV, v.S, v.F, B,
                       g_log2);
  else
    hipLaunchKernelGGL((k_sddmm<T, CH, false>), grid, dim3(MP_THREADS), 0, s, v.ptr, v.idx,
                       v.part_seg, v.part_nz, (const T*)dY, (const T*)X, (T*)dV, v.S, v.F, B,
                       g_log2);
}

template <typename T>
static void launch_sddmm_dt(const seg_view& v, const void* dY, const void* X, snack_layout lay,
                            int32_t B, void* dV, const lane_shape& sh, hipStream_t s) {
  switch (sh.ch) {
    case 1: launch_sddmm_ch<T, 1>(v, dY, X, lay, B, dV, sh.g_log2, s); break;
    case 2: launch_sddmm_ch<T, 2>(v, dY, X, lay, B, dV, sh.g_log2, s); break;
    case 4: launch_sddmm_ch<T, 4>(v, dY, X, lay, B, dV, sh.g_log2, s); break;
    default:
      if constexpr (sizeof(T) == 2) launch_sddmm_ch<T, 8>(v, dY, X, lay, B, dV, sh.g_log2, s);
      break;
  }
}

snack_status launch_sddmm(const seg_view& v, const void* dY, const void* X, snack_dtype dt,
                          snack_layout lay, int32_t B, void* dV, hipStream_t s) {
  if (v.nnz == 0) return SNACK_OK;
  if (B == 0) {
    dim3 g((unsigned)cdiv(v.nnz, 256));
    if (dt == SNACK_F32) hipLaunchKernelGGL(k_fill_zero<float>, g, dim3(256), 0, s, (float*)dV, v.nnz);
    else hipLaunchKernelGGL(k_fill_zero<bf16>, g, dim3(256), 0, s, (bf16*)dV, v.nnz);
    return hipGetLastError() == hipSuccess ? SNACK_OK : SNACK_E_HIP;
  }
  lane_shape sh = pick_shape(dt, B);
  if (dt == SNACK_F32) launch_sddmm_dt<float>(v, dY, X, lay, B, dV, sh, s);
  else launch_sddmm_dt<bf16>(v, dY, X, lay, B, dV, sh, s);
  return hipGetLastError() == hipSuccess ? SNACK_OK : SNACK_E_HIP;
}

}  // namespace snk
