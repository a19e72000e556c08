// wave.h -- device helpers of the wave-per-segment kernels (one 64-lane wave
// owns a whole segment): segment lookup, batched entry loads, gather-round
// groups and the butterfly reduce-scatter.
#pragma once

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace snk {

constexpr int WV_THREADS = 256;  // four waves per workgroup, one segment each
constexpr int WV_U = 4;          // index/value loads of 64 entries kept in flight

// Segment handled by this wave; blocks are spread over the dies so that each
// die covers one contiguous range when xcd_blocks > 0.
__device__ __forceinline__ int32_t wave_segment(int32_t xcd_blocks) {
  const int32_t blk = xcd_blocks > 0
                          ? (int32_t)(blockIdx.x % NUM_XCD) * xcd_blocks +
                                (int32_t)(blockIdx.x / NUM_XCD)
                          : (int32_t)blockIdx.x;
  return __builtin_amdgcn_readfirstlane(blk * (WV_THREADS / SNK_WAVE) +
                                        (int32_t)(threadIdx.x / SNK_WAVE));
}

// Butterfly reduce-scatter of acc[CH] over the lanes that share (lane mod
// LPE): after the call, lane l holds in acc[0] the total of batch column
// col_of(l) of its LPE group, where that column's bits come from lane bits
// 5, 4, ... (most significant first).  CH <= 64 / LPE.
template <int CH, int LPE>
__device__ __forceinline__ int reduce_scatter(float (&acc)[CH], int lane) {
  int c = 0;
  int o = 32;
#pragma unroll
  for (int n = CH; n > 1; n >>= 1, o >>= 1) {
    const bool up = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const float send = up ? acc[i] : acc[i + n / 2];
      const float keep = up ? acc[i + n / 2] : acc[i];
      acc[i] = keep + __shfl_xor(send, o, SNK_WAVE);
    }
    if (up) c += n / 2;
  }
#pragma unroll
  for (; o >= LPE; o >>= 1) acc[0] += __shfl_xor(acc[0], o, SNK_WAVE);
  return c;
}

// x <- 0 where !ok, on the raw words of a gathered chunk (an entry past the
// segment's end was gathered at a valid, clamped address and must not add
// even an Inf or NaN of that row).
template <typename T, int CH>
__device__ __forceinline__ void zero_unless(vec<T, CH>& x, bool ok) {
  constexpr int W = (int)(CH * sizeof(T) + 3) / 4;
  if constexpr (CH * sizeof(T) >= 4) {
    uint32_t* w = reinterpret_cast<uint32_t*>(&x);
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = ok ? w[i] : 0u;
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) x.v[c] = ok ? x.v[c] : (T)0;
  }
}

// Loads entries base + q*64 + lane (q < WV_U) with their index clamped to the
// segment's last entry, so that every load is unconditional and all of them
// are in flight together.  Values past the end are 0; with PERM, pk receives
// each entry's value position.  vals is not restrict-qualified: the fused
// backward writes the same array after these loads.
template <typename T, bool PERM, bool VALS, int U = WV_U>
__device__ __forceinline__ void load_entries(const int32_t* __restrict__ idx,
                                             const int32_t* __restrict__ perm, const T* vals,
                                             int32_t base, int32_t e, int lane,
                                             int32_t (&ci)[U], float (&cv)[U],
                                             int32_t (&pk)[U]) {
  int32_t kc[U];
#pragma unroll
  for (int q = 0; q < U; ++q) kc[q] = min(base + q * SNK_WAVE + lane, e - 1);
#pragma unroll
  for (int q = 0; q < U; ++q) ci[q] = idx[kc[q]];
  if constexpr (VALS) {
    T raw[U];
    if constexpr (PERM) {
#pragma unroll
      for (int q = 0; q < U; ++q) pk[q] = perm[kc[q]];
#pragma unroll
      for (int q = 0; q < U; ++q) raw[q] = vals[pk[q]];
    } else {
#pragma unroll
      for (int q = 0; q < U; ++q) raw[q] = vals[kc[q]];
    }
#pragma unroll
    for (int q = 0; q < U; ++q)
      cv[q] = (base + q * SNK_WAVE + lane < e) ? elem<T>::to_f(raw[q]) : 0.f;
  }
}

// Gather rounds issued together before any is consumed: at most 16 (one
// gathered chunk each per lane), never more than one loaded batch of U
// 64-entry chunks holds.
template <int LPE, int U = WV_U>
constexpr int wave_rg() {
  return U * LPE < 16 ? U * LPE : 16;
}

// 64-entry chunks per loaded batch for segments longer than one batch of
// WV_U chunks: with few lanes per entry a round covers many entries, so the
// batch grows to 16 rounds (1,024 entries at one lane per entry) and a long
// segment takes fewer dependent load/gather round trips.
template <int LPE>
constexpr int wave_u_long() {
  return LPE >= 4 ? WV_U : 16 / LPE;
}

// Calls f(integral_constant<N>) for the runtime n in [1, NMAX], so that a
// round group runs straight-line code with no exit inside (the compiler
// sinks gathers into conditional blocks and waits for each there).
template <int NMAX, typename F>
__device__ __forceinline__ void with_count(int n, F&& f) {
  if constexpr (NMAX >= 1) {
    if (n >= NMAX) f(std::integral_constant<int, NMAX>{});
    else with_count<NMAX - 1>(n, f);
  }
}

// NR gather rounds of EPI entries each, from the loaded chunks ci/cv (round i
// takes chunk i / LPE, lanes (i % LPE) * EPI + slot): the activation chunk
// of each round's entry and its value.  Only the last round can hold entries
// past the end e; their chunks are zeroed.
template <typename T, int CH, int LPE, int NR>
__device__ __forceinline__ void gather_rounds(const T* __restrict__ xb, int32_t B,
                                              const int32_t* ci, const float* cv, int32_t rb,
                                              int32_t e, int slot, vec<T, CH> (&xv)[NR],
                                              float (&vj)[NR]) {
  constexpr int EPI = SNK_WAVE / LPE;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int q = i / LPE, src = (i % LPE) * EPI + slot;
    const int32_t cj = LPE == 1 ? ci[q] : __shfl(ci[q], src, SNK_WAVE);
    vj[i] = LPE == 1 ? cv[q] : __shfl(cv[q], src, SNK_WAVE);
    xv[i] = *reinterpret_cast<const vec<T, CH>*>(xb + (int64_t)cj * B);
  }
  zero_unless<T, CH>(xv[NR - 1], rb + (NR - 1) * EPI + slot < e);
}

// acc[c] += sum_i vj[i] * xv[i][c].  bf16: rounds i and i+1 together in one
// v_dot2_f32_bf16 per column; the pairs (x_i[c], x_i+1[c]) come from one byte
// permute of the two gathered words (a bf16 value v is the high half of its
// fp32 widening, so (v_i, v_i+1) is a permute too).
template <typename T, int CH, int NR>
__device__ __forceinline__ void accumulate_rounds(const vec<T, CH> (&xv)[NR],
                                                  const float (&vj)[NR], float (&acc)[CH]) {
  if constexpr (sizeof(T) == 2 && CH >= 2) {
    typedef __bf16 __attribute__((ext_vector_type(2))) bf2;
#pragma unroll
    for (int i = 0; i < NR; i += 2) {
      const bool two = i + 1 < NR;
      const uint32_t va = __float_as_uint(vj[i]);
      const uint32_t vb = two ? __float_as_uint(vj[i + 1]) : 0u;
      const uint32_t vp = __builtin_amdgcn_perm(vb, va, 0x07060302u);
      const uint32_t* wa = reinterpret_cast<const uint32_t*>(&xv[i]);
      const uint32_t* wb = reinterpret_cast<const uint32_t*>(&xv[two ? i + 1 : i]);
#pragma unroll
      for (int w = 0; w < CH / 2; ++w) {
        const uint32_t b = two ? wb[w] : 0u;
        const uint32_t lo = __builtin_amdgcn_perm(b, wa[w], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(b, wa[w], 0x07060302u);
        acc[2 * w] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, vp),
                                                     __builtin_bit_cast(bf2, lo), acc[2 * w],
                                                     false);
        acc[2 * w + 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, vp),
                                                         __builtin_bit_cast(bf2, hi),
                                                         acc[2 * w + 1], false);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
#pragma unroll
      for (int c = 0; c < CH; ++c) acc[c] = fmaf(vj[i], elem<T>::to_f(xv[i].v[c]), acc[c]);
    }
  }
}

// Every gather of NR rounds first, then the FMAs.
template <typename T, int CH, int LPE, int NR>
__device__ __forceinline__ void spmm_rounds(const T* __restrict__ xb, int32_t B,
                                            const int32_t* ci, const float* cv, int32_t rb,
                                            int32_t e, int slot, float (&acc)[CH]) {
  vec<T, CH> xv[NR];
  float vj[NR];
  gather_rounds<T, CH, LPE, NR>(xb, B, ci, cv, rb, e, slot, xv, vj);
  accumulate_rounds<T, CH, NR>(xv, vj, acc);
}

// Sums each round's partial dot over the LPE lanes of its slot, then permutes
// so that lane l of chunk q holds the result of entry q*64 + l (rounds past
// NR give 0).
template <int LPE, int NR>
__device__ __forceinline__ void reduce_permute(const float (&part)[NR], int lane,
                                               float (&out)[(NR + LPE - 1) / LPE]) {
  constexpr int EPI = SNK_WAVE / LPE;
  constexpr int NQ = (NR + LPE - 1) / LPE;
  float res[NQ * LPE];
#pragma unroll
  for (int i = 0; i < NQ * LPE; ++i) {
    float d = 0.f;
    if (i < NR) {
      d = part[i];
#pragma unroll
      for (int off = 1; off < LPE; off <<= 1) d += __shfl_xor(d, off, SNK_WAVE);
    }
    res[i] = d;
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    // entry q*64 + lane was dotted in round lane / EPI by slot lane % EPI
    out[q] = res[q * LPE];
    if constexpr (LPE > 1) {
      const int from = (lane % EPI) * LPE;
#pragma unroll
      for (int j = 0; j < LPE; ++j) {
        const float v = __shfl(res[q * LPE + j], from, SNK_WAVE);
        if (lane / EPI == j) out[q] = v;
      }
    }
  }
}

// The dot of each round's gathered chunk with g, summed over the LPE lanes
// of its slot and permuted to lane = entry (reduce_permute).
template <typename T, int CH, int LPE, int NR>
__device__ __forceinline__ void round_dots(const vec<T, CH> (&xv)[NR], const vec<T, CH>& g,
                                           int lane, float (&out)[(NR + LPE - 1) / LPE]) {
  float part[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) part[i] = dot_acc<T, CH>(g, xv[i], 0.f);
  reduce_permute<LPE, NR>(part, lane, out);
}

// ---- LDS staging of the gathered input (shared by the products, the value
// gradient and the fused backward): views whose whole node-major input fits
// a workgroup's LDS copy it once per 16-wave workgroup and gather from LDS.
constexpr int WL_THREADS = 1024;
// gfx950 gives a workgroup up to 160 KB of LDS (the CU's whole LDS): inputs
// above half of it run one workgroup per CU, smaller ones two.  With one
// workgroup per CU only one lane per entry pays off (measured: 8192^2 at
// B=8 and the LLaMA up input gradient at B=4 11-32% faster, the LLaMA down
// input gradient at B=16, two lanes per entry, 9% slower).
constexpr int WL_LDS = 160 * 1024;
inline int32_t wave_lds_blocks(int64_t x_bytes, int32_t S) {
  const int64_t per_cu = x_bytes > WL_LDS / 2 ? 1 : 2;
  return (int32_t)std::min<int64_t>(per_cu * 256, cdiv(S, WL_THREADS / SNK_WAVE));
}
constexpr int WL_MIN_SEGMENTS = 16384;
// Fewer segments still take the LDS path when the input is large enough
// that the gathers miss the L1 cache often and segments are long enough
// (>= 256 entries on average) to amortise the staging.  Measured: the
// LLaMA-shaped column views' input gradient 10-22% faster (22-32 KB
// inputs); at 16 KB (8192^2, batch 1) the value gradient 18% faster but the
// products 5% slower, hence the two sizes; inputs of a few KB (4096^2 at
// batch 1) and short segments (4096^2 at batch 8) lose to the cached gathers.
constexpr int WL_MID_SEGMENTS = 2048;
constexpr int64_t WL_MID_BYTES_SPMM = 20 * 1024;
constexpr int64_t WL_MID_BYTES_SDDMM = 16 * 1024;
constexpr int64_t WL_MID_AVG = 256;

// Whether a view takes the LDS-staged kernels (one batch pass and no split
// segment are checked by the caller); mid_bytes: the product's input-size
// bound for views of fewer than WL_MIN_SEGMENTS segments.
inline bool wave_lds_fits(const seg_view& v, int64_t x_bytes, const void* Xt,
                          int64_t mid_bytes, int lpe) {
  if (x_bytes > WL_LDS || (uintptr_t)Xt % 16 != 0) return false;
  if (x_bytes > WL_LDS / 2 && lpe > 1) return false;
  if (v.S >= WL_MIN_SEGMENTS) return true;
  return v.S >= WL_MID_SEGMENTS && x_bytes >= mid_bytes && v.nnz >= WL_MID_AVG * v.S;
}

struct wave_shape {
  int ch;   // batch columns per lane
  int lpe;  // lanes per entry
};

// Widest lane chunk dividing B (16-byte gathers at most), then the fewest
// lanes per entry that cover the batch, capped at 64 batch columns per pass.
inline wave_shape wave_pick(snack_dtype dt, int32_t B) {
  const int chmax = dt == SNACK_BF16 ? 8 : 4;
  int ch = 1;
  while (ch < chmax && B % (ch * 2) == 0) ch *= 2;
  int lpe = 1;
  while (lpe * ch < B && lpe * ch < 64) lpe *= 2;
  return {ch, lpe};
}

}  // namespace snk
