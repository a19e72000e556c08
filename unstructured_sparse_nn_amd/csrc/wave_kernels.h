// wave_kernels.h -- the wave-per-segment kernels and their launch templates,
// instantiated per element type by wave_spmm_*.hip and wave_sddmm_*.hip.
//
// One 64-lane wave per output segment (row, or column for the transpose);
// segments of a tile or more are summed as tile pieces by the first
// workgroups of the same launch (k_wave_spmm_split, k_wave_sddmm_split); the
// products' pieces are finished by the fix-up of spmm.hip.
//
// The same three products as spmm.hip ("Beyond Masked Sparsity: SNACK
// Enables Truly Sparse Neural Networks on GPU", Abstract: compute only the
// nonzero connections, forward and backward):
//   out[b, s] = sum_{k in segment s} v[k] * in[b, idx[k]]    (k_wave_spmm)
//   dV[k]     = sum_b dY[b, s(k)] * X[b, idx[k]]             (k_wave_sddmm)
// but with one 64-lane wave owning a whole segment, so there is no merge-path
// search, no segment bookkeeping per entry, no LDS staging and no barrier.
// What a wave does per segment:
//   * the segment's bounds come in through scalar loads (wave-uniform);
//   * its indices and values are read 64 entries per load, coalesced, four
//     loads in flight (up to sixteen for long segments at one or two lanes
//     per entry);
//   * lanes are split into EPI = 64 / LPE entry slots of LPE lanes; each lane
//     owns CH consecutive batch columns, so one round gathers the node-major
//     activation rows of EPI entries (LPE * CH * elem bytes per entry);
//   * the index and value of each slot's entry come from the loading lane by
//     a cross-lane permute;
//   * at the end, the EPI partial sums of each batch column are added by a
//     butterfly reduce-scatter: each exchange step halves the values a lane
//     holds, CH - 1 + log2(EPI / CH) shuffles in all instead of CH log2(EPI).
// A fixed reduction tree: results are bitwise reproducible.  Measured with
// rocprofv3 at 4096^2, 95%, batch 32 bf16: the merge-path kernel issued 4.7
// VALU (and 4.4 SALU) wave instructions per stored entry; this one issues
// 1.8 VALU and 0.3 SALU.
#pragma once

#include <climits>
#include <cstdlib>

#include "common.h"
#include "internal.h"
#include "wave.h"

namespace snk {

// acc[c] = sum over entries [a, e) of v * in[idx, b0 + c]: batches of four
// 64-entry loads, each split into round groups of straight-line code.
template <typename T, int CH, int LPE, bool PERM, int U>
__device__ __forceinline__ void spmm_batches(const int32_t* __restrict__ idx,
                                             const int32_t* __restrict__ perm, const T* vals,
                                             const T* __restrict__ xb, int32_t B, int32_t a,
                                             int32_t e, int lane, int slot, float (&acc)[CH]) {
  constexpr int EPI = SNK_WAVE / LPE;
  constexpr int RG = wave_rg<LPE, U>();  // rounds per group (a whole number of chunks)
  for (int32_t base = a; base < e; base += U * SNK_WAVE) {
    int32_t ci[U], pk[U];
    float cv[U];
    load_entries<T, PERM, true, U>(idx, perm, vals, base, e, lane, ci, cv, pk);
#pragma unroll
    for (int g = 0; g < U * LPE / RG; ++g) {
      const int q0 = g * RG / LPE;
      const int32_t rb = base + g * RG * EPI;  // first entry of the group (wave-uniform)
      if (rb >= e) break;
      const int nr = (e - rb + EPI - 1) / EPI;
      with_count<RG>(nr, [&](auto n) {
        spmm_rounds<T, CH, LPE, decltype(n)::value>(xb, B, ci + q0, cv + q0, rb, e, slot, acc);
      });
    }
  }
}

template <typename T, int CH, int LPE, bool PERM>
__device__ __forceinline__ void spmm_range(const int32_t* __restrict__ idx,
                                           const int32_t* __restrict__ perm, const T* vals,
                                           const T* __restrict__ xb, int32_t B, int32_t a,
                                           int32_t e, int lane, int slot, float (&acc)[CH]) {
  constexpr int UL = wave_u_long<LPE>();
#pragma unroll
  for (int c = 0; c < CH; ++c) acc[c] = 0.f;
  if (UL > WV_U && e - a > WV_U * SNK_WAVE)  // wave-uniform: a long segment, larger batches
    spmm_batches<T, CH, LPE, PERM, UL>(idx, perm, vals, xb, B, a, e, lane, slot, acc);
  else
    spmm_batches<T, CH, LPE, PERM, WV_U>(idx, perm, vals, xb, B, a, e, lane, slot, acc);
}

// The tile pieces of split segments (segments of >= T entries, cut by the
// load-balanced tiles), one wave per tile p, summed into the carry slots
// that k_fixup adds in tile order:
//   carry[p]     the piece of the segment that continues into tile p+1
//                (cut p+1 is inside it): from the tile's start, or from the
//                segment's start if it begins in this tile, to cut p+1;
//   carry[P + p] the last piece of the segment cut at p: from cut p to its end.
// Pieces are at most 2T entries, so no wave serialises a long segment.
template <typename T, int CH, int LPE, bool PERM>
__device__ __forceinline__ void wave_pieces_of(
    int32_t p, const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm, const T* __restrict__ vals,
    const int32_t* __restrict__ part_seg, const int32_t* __restrict__ part_nz,
    const int32_t* __restrict__ cut, const T* __restrict__ Xt, float* __restrict__ carry,
    int32_t P, int32_t B) {
  constexpr int EPI = SNK_WAVE / LPE;
  constexpr int LOW = EPI / CH;
  if (p >= P) return;
  const int32_t s0 = part_seg[p], s1 = part_seg[p + 1];
  const bool c0 = cut[p] != 0, c1 = cut[p + 1] != 0;
  const bool last_piece = c0 && !(c1 && s1 == s0);
  if (!c1 && !last_piece) return;
  const int lane = lane_id();
  const int slot = lane / LPE;
  const int sub = lane % LPE;
  const int32_t b0 = (int32_t)blockIdx.y * (LPE * CH) + sub * CH;
  const bool bvalid = b0 < B;
  const T* __restrict__ xb = Xt + (bvalid ? b0 : 0);
  auto piece = [&](int32_t a, int32_t e, float* __restrict__ dst) {
    float acc[CH];
    spmm_range<T, CH, LPE, PERM>(idx, perm, vals, xb, B, a, e, lane, slot, acc);
    const int c = reduce_scatter<CH, LPE>(acc, lane);
    if ((slot % LOW) == 0 && bvalid) dst[b0 + c] = acc[0];
  };
  if (last_piece) piece(part_nz[p], ptr[s0 + 1], carry + ((int64_t)P + p) * B);
  if (c1) piece((c0 && s0 == s1) ? part_nz[p] : ptr[s1], part_nz[p + 1], carry + (int64_t)p * B);
}

// Segment s of the pass blockIdx.y (batch columns b0 = blockIdx.y * LPE * CH
// + ...).  The gathered rows are read from Xs with row stride xstride, Xs
// holding the batch columns from xcol0 on: the node-major input itself
// (xstride = B, xcol0 = 0) or a copy of it, or of the pass's columns, in LDS.
template <typename T, int CH, int LPE, bool PERM, bool NODE_OUT, int ACT>
__device__ __forceinline__ void wave_spmm_of(
    int32_t s, const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm, const T* __restrict__ vals, const T* __restrict__ Xs,
    T* __restrict__ Y, int32_t S, int32_t B, int32_t long_len, int32_t xstride,
    int32_t xcol0 = 0) {
  constexpr int EPI = SNK_WAVE / LPE;  // entries per gather round
  static_assert(CH <= EPI, "reduce-scatter needs CH <= 64 / LPE");
  if (s >= S) return;
  const int lane = lane_id();
  const int slot = lane / LPE;
  const int sub = lane % LPE;
  const int32_t b0 = (int32_t)blockIdx.y * (LPE * CH) + sub * CH;
  const bool bvalid = b0 < B;
  // lanes past the batch read the first column
  const T* __restrict__ xb = Xs + (bvalid ? b0 - xcol0 : 0);
  const int32_t a = ptr[s], e = ptr[s + 1];

  if (e - a >= long_len) return;  // a split segment: its tile pieces are summed elsewhere

  float acc[CH];
  spmm_range<T, CH, LPE, PERM>(idx, perm, vals, xb, xstride, a, e, lane, slot, acc);
  const int c = reduce_scatter<CH, LPE>(acc, lane);
  // lanes whose slot bits below the scattered ones are zero write
  constexpr int LOW = EPI / CH;  // slot values sharing one column after the scatter
  if ((slot % LOW) == 0 && bvalid) {
    const float r = apply_act(acc[0], ACT);
    const int32_t b = b0 + c;
    if constexpr (NODE_OUT) Y[(int64_t)s * B + b] = elem<T>::from_f(r);
    else Y[(int64_t)b * S + s] = elem<T>::from_f(r);
  }
}

template <typename T, int CH, int LPE, bool PERM, bool NODE_OUT, int ACT>
__global__ __launch_bounds__(WV_THREADS) void k_wave_spmm(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm, const T* __restrict__ vals, const T* __restrict__ Xt,
    T* __restrict__ Y, int32_t S, int32_t B, int32_t xcd_blocks, int32_t long_len) {
  wave_spmm_of<T, CH, LPE, PERM, NODE_OUT, ACT>(wave_segment(xcd_blocks), ptr, idx, perm, vals,
                                                Xt, Y, S, B, long_len, B);
}

// Layers whose whole node-major input fits in LDS (F * B elements of at most
// WL_LDS bytes: batch 1 up to 32,768 bf16 features) and has many segments:
// each 16-wave workgroup copies the input into LDS once (16-byte copies, one
// barrier), then its waves take segments in a grid-stride loop and gather
// from LDS.  On large layers the gathers are otherwise scattered L2 requests
// (one per entry at batch 1), which bound the launch well below the entry
// stream; from LDS they cost a few LDS cycles per 64 entries.  One batch pass
// (B <= LPE * CH); no split segments.
template <typename T, int CH, int LPE, bool PERM, bool NODE_OUT, int ACT>
__global__ __launch_bounds__(WL_THREADS) void k_wave_spmm_lds(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm, const T* __restrict__ vals, const T* __restrict__ Xt,
    T* __restrict__ Y, int32_t S, int32_t B, int64_t x_elems) {
  extern __shared__ uint4 xs_raw[];
  const int64_t nbytes = x_elems * (int64_t)sizeof(T);
  const int64_t n16 = nbytes / 16;  // whole 16-byte words (Xt is 16-byte aligned)
  const uint4* __restrict__ src = reinterpret_cast<const uint4*>(Xt);
  for (int64_t i = threadIdx.x; i < n16; i += WL_THREADS) xs_raw[i] = src[i];
  T* xs = reinterpret_cast<T*>(xs_raw);
  for (int64_t i = n16 * (16 / (int64_t)sizeof(T)) + threadIdx.x; i < x_elems; i += WL_THREADS)
    xs[i] = Xt[i];  // the tail past the last whole word
  __syncthreads();
  const int32_t waves = (int32_t)gridDim.x * (WL_THREADS / SNK_WAVE);
  for (int32_t s = __builtin_amdgcn_readfirstlane((int32_t)blockIdx.x * (WL_THREADS / SNK_WAVE) +
                                                  (int32_t)(threadIdx.x / SNK_WAVE));
       s < S; s += waves)
    wave_spmm_of<T, CH, LPE, PERM, NODE_OUT, ACT>(s, ptr, idx, perm, vals, xs, Y, S, B,
                                                  INT32_MAX, B);
}

// Both halves of a view with split segments in one launch, so that they
// overlap: workgroups below pblk (a multiple of NUM_XCD) run the tile pieces
// (wave_pieces_of), the rest the segments of < long_len entries (as
// k_wave_spmm, in the same die-contiguous order, which a multiple of NUM_XCD
// keeps).
template <typename T, int CH, int LPE, bool PERM, bool NODE_OUT, int ACT>
__global__ __launch_bounds__(WV_THREADS) void k_wave_spmm_split(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm, const T* __restrict__ vals, const T* __restrict__ Xt,
    T* __restrict__ Y, int32_t S, int32_t B, int32_t xcd_blocks, int32_t long_len,
    const int32_t* __restrict__ part_seg, const int32_t* __restrict__ part_nz,
    const int32_t* __restrict__ cut, float* __restrict__ carry, int32_t P, int32_t pblk) {
  const int32_t w = (int32_t)(threadIdx.x / SNK_WAVE);
  const int32_t bx = (int32_t)blockIdx.x;
  if (bx < pblk) {
    const int32_t p = __builtin_amdgcn_readfirstlane(bx * (WV_THREADS / SNK_WAVE) + w);
    wave_pieces_of<T, CH, LPE, PERM>(p, ptr, idx, perm, vals, part_seg, part_nz, cut, Xt, carry,
                                     P, B);
    return;
  }
  const int32_t sb = bx - pblk;
  const int32_t blk = xcd_blocks > 0 ? (sb % NUM_XCD) * xcd_blocks + sb / NUM_XCD : sb;
  const int32_t s = __builtin_amdgcn_readfirstlane(blk * (WV_THREADS / SNK_WAVE) + w);
  wave_spmm_of<T, CH, LPE, PERM, NODE_OUT, ACT>(s, ptr, idx, perm, vals, Xt, Y, S, B, long_len,
                                                B);
}

// The value gradient of NR rounds.  One batch pass (B <= LPE * CH): every
// gather first, then the dots.  Wider batches: per pass of LPE * CH columns,
// the row's dY chunk and the NR gathered X chunks, their dots accumulated;
// then the LPE-lane sums and, per chunk of 64 entries, one coalesced store.
template <typename T, int CH, int LPE, int NR, bool MULTI>
__device__ __forceinline__ void sddmm_rounds(const T* __restrict__ Xt,
                                             const T* __restrict__ dYrow, int32_t B,
                                             int32_t passes, int32_t b0, const int32_t* ci,
                                             int32_t rb, int32_t e, int lane, int slot,
                                             T* __restrict__ dV) {
  constexpr int EPI = SNK_WAVE / LPE;
  constexpr int NQ = (NR + LPE - 1) / LPE;
  int32_t cj[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int q = i / LPE, src = (i % LPE) * EPI + slot;
    cj[i] = LPE == 1 ? ci[q] : __shfl(ci[q], src, SNK_WAVE);
  }
  float part[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) part[i] = 0.f;
  if (!MULTI) passes = 1;  // one pass: straight-line code
  for (int32_t bp = 0; bp < passes; ++bp) {
    const int32_t b = bp * (LPE * CH) + b0;
    const bool ok = b < B;
    const int32_t bb = ok ? b : 0;  // lanes past the batch read column 0 and add nothing
    vec<T, CH> g = *reinterpret_cast<const vec<T, CH>*>(dYrow + bb);
    zero_unless<T, CH>(g, ok);
    vec<T, CH> xv[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i)
      xv[i] = *reinterpret_cast<const vec<T, CH>*>(Xt + (int64_t)cj[i] * B + bb);
#pragma unroll
    for (int i = 0; i < NR; ++i) part[i] = dot_acc<T, CH>(g, xv[i], part[i]);
  }
  float out[NQ];
  reduce_permute<LPE, NR>(part, lane, out);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int32_t k = rb + q * SNK_WAVE + lane;
    if (k < e) dV[k] = elem<T>::from_f(out[q]);
  }
}

// dV[k] for the entries [a, e) of segment s: each round gathers EPI entries'
// X chunks and dots them with the segment's dY chunk, the LPE lanes of a
// slot add their partial dots, and every 64 entries the results are
// permuted to lane = entry and stored coalesced.
template <typename T, int CH, int LPE, bool MULTI, int U>
__device__ __forceinline__ void sddmm_batches(const int32_t* __restrict__ idx,
                                              const T* __restrict__ dYrow,
                                              const T* __restrict__ Xt, int32_t B,
                                              int32_t passes, int32_t a, int32_t e, int lane,
                                              int slot, int32_t b0, T* __restrict__ dV) {
  constexpr int EPI = SNK_WAVE / LPE;
  constexpr int RG = wave_rg<LPE, U>();
  for (int32_t base = a; base < e; base += U * SNK_WAVE) {
    int32_t ci[U], unused_pk[U];
    float unused[U];
    load_entries<T, false, false, U>(idx, nullptr, (const T*)nullptr, base, e, lane, ci, unused,
                                     unused_pk);
#pragma unroll
    for (int gi = 0; gi < U * LPE / RG; ++gi) {
      const int q0 = gi * RG / LPE;
      const int32_t rb = base + gi * RG * EPI;
      if (rb >= e) break;
      const int nr = (e - rb + EPI - 1) / EPI;
      with_count<RG>(nr, [&](auto n) {
        sddmm_rounds<T, CH, LPE, decltype(n)::value, MULTI>(Xt, dYrow, B, passes, b0, ci + q0,
                                                            rb, e, lane, slot, dV);
      });
    }
  }
}

template <typename T, int CH, int LPE, bool MULTI>
__device__ __forceinline__ void sddmm_range(const int32_t* __restrict__ idx,
                                            const T* __restrict__ dYt,
                                            const T* __restrict__ Xt, int32_t B, int32_t s,
                                            int32_t a, int32_t e, int lane, int slot, int32_t b0,
                                            T* __restrict__ dV) {
  constexpr int UL = wave_u_long<LPE>();
  const int32_t passes = (B + LPE * CH - 1) / (LPE * CH);
  const T* __restrict__ dYrow = dYt + (int64_t)s * B;
  if (UL > WV_U && e - a > WV_U * SNK_WAVE)  // wave-uniform: a long segment, larger batches
    sddmm_batches<T, CH, LPE, MULTI, UL>(idx, dYrow, Xt, B, passes, a, e, lane, slot, b0, dV);
  else
    sddmm_batches<T, CH, LPE, MULTI, WV_U>(idx, dYrow, Xt, B, passes, a, e, lane, slot, b0, dV);
}

// One row per wave; rows of >= long_len entries (split by the tiles) are
// left to the tile pieces (wave_sddmm_pieces_of).  Batches wider than
// LPE * CH run in passes.
template <typename T, int CH, int LPE, bool MULTI>
__device__ __forceinline__ void wave_sddmm_of(int32_t s, const int32_t* __restrict__ ptr,
                                              const int32_t* __restrict__ idx,
                                              const T* __restrict__ dYt,
                                              const T* __restrict__ Xt, T* __restrict__ dV,
                                              int32_t S, int32_t B, int32_t long_len) {
  if (s >= S) return;
  const int lane = lane_id();
  const int slot = lane / LPE;
  const int32_t b0 = (lane % LPE) * CH;
  const int32_t a = ptr[s], e = ptr[s + 1];
  if (a == e || e - a >= long_len) return;
  sddmm_range<T, CH, LPE, MULTI>(idx, dYt, Xt, B, s, a, e, lane, slot, b0, dV);
}

template <typename T, int CH, int LPE, bool MULTI>
__global__ __launch_bounds__(WV_THREADS) void k_wave_sddmm(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const T* __restrict__ dYt, const T* __restrict__ Xt, T* __restrict__ dV, int32_t S,
    int32_t B, int32_t long_len) {
  wave_sddmm_of<T, CH, LPE, MULTI>(wave_segment(0), ptr, idx, dYt, Xt, dV, S, B, long_len);
}

// The tile pieces of split rows, one wave per tile (the same pieces as
// wave_pieces_of); each entry's dV is final, so no carry is needed.
template <typename T, int CH, int LPE, bool MULTI>
__device__ __forceinline__ void wave_sddmm_pieces_of(
    int32_t p, const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ part_seg, const int32_t* __restrict__ part_nz,
    const int32_t* __restrict__ cut, const T* __restrict__ dYt, const T* __restrict__ Xt,
    T* __restrict__ dV, int32_t P, int32_t B) {
  if (p >= P) return;
  const int32_t s0 = part_seg[p], s1 = part_seg[p + 1];
  const bool c0 = cut[p] != 0, c1 = cut[p + 1] != 0;
  const bool last_piece = c0 && !(c1 && s1 == s0);
  if (!c1 && !last_piece) return;
  const int lane = lane_id();
  const int slot = lane / LPE;
  const int32_t b0 = (lane % LPE) * CH;
  if (last_piece)
    sddmm_range<T, CH, LPE, MULTI>(idx, dYt, Xt, B, s0, part_nz[p], ptr[s0 + 1], lane, slot, b0,
                                   dV);
  if (c1)
    sddmm_range<T, CH, LPE, MULTI>(idx, dYt, Xt, B, s1, (c0 && s0 == s1) ? part_nz[p] : ptr[s1],
                                   part_nz[p + 1], lane, slot, b0, dV);
}

// The value gradient with the whole node-major X in LDS (the conditions of
// k_wave_spmm_lds): X staged once per 16-wave workgroup, rows taken in a
// grid-stride loop, each entry's X chunk read from LDS; the row's dY chunk
// is read from memory as in k_wave_sddmm.
template <typename T, int CH, int LPE>
__global__ __launch_bounds__(WL_THREADS) void k_wave_sddmm_lds(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const T* __restrict__ dYt, const T* __restrict__ Xt, T* __restrict__ dV, int32_t S,
    int32_t B, int64_t x_elems) {
  extern __shared__ uint4 xs_raw[];
  const int64_t n16 = x_elems * (int64_t)sizeof(T) / 16;
  const uint4* __restrict__ src = reinterpret_cast<const uint4*>(Xt);
  for (int64_t i = threadIdx.x; i < n16; i += WL_THREADS) xs_raw[i] = src[i];
  T* xs = reinterpret_cast<T*>(xs_raw);
  for (int64_t i = n16 * (16 / (int64_t)sizeof(T)) + threadIdx.x; i < x_elems; i += WL_THREADS)
    xs[i] = Xt[i];
  __syncthreads();
  const int32_t waves = (int32_t)gridDim.x * (WL_THREADS / SNK_WAVE);
  for (int32_t s = __builtin_amdgcn_readfirstlane((int32_t)blockIdx.x * (WL_THREADS / SNK_WAVE) +
                                                  (int32_t)(threadIdx.x / SNK_WAVE));
       s < S; s += waves)
    wave_sddmm_of<T, CH, LPE, false>(s, ptr, idx, dYt, xs, dV, S, B, INT32_MAX);
}

// Both halves of a view with split rows in one launch, so that they overlap:
// workgroups below pblk run the tile pieces, the rest the rows of < long_len
// entries.
template <typename T, int CH, int LPE, bool MULTI>
__global__ __launch_bounds__(WV_THREADS) void k_wave_sddmm_split(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ part_seg, const int32_t* __restrict__ part_nz,
    const int32_t* __restrict__ cut, const T* __restrict__ dYt, const T* __restrict__ Xt,
    T* __restrict__ dV, int32_t S, int32_t P, int32_t B, int32_t long_len, int32_t pblk) {
  const int32_t w = (int32_t)(threadIdx.x / SNK_WAVE);
  const int32_t bx = (int32_t)blockIdx.x;
  if (bx < pblk) {
    const int32_t p = __builtin_amdgcn_readfirstlane(bx * (WV_THREADS / SNK_WAVE) + w);
    wave_sddmm_pieces_of<T, CH, LPE, MULTI>(p, ptr, idx, part_seg, part_nz, cut, dYt, Xt, dV, P,
                                            B);
    return;
  }
  const int32_t s = __builtin_amdgcn_readfirstlane((bx - pblk) * (WV_THREADS / SNK_WAVE) + w);
  wave_sddmm_of<T, CH, LPE, MULTI>(s, ptr, idx, dYt, Xt, dV, S, B, long_len);
}

// ---------------------------------------------------------------- launch templates
// Segments of >= T entries (split view) are skipped by the per-segment
// kernel, summed piecewise per tile into the carry slots, and finished by
// k_fixup.
template <typename T, int CH, int LPE, bool PERM, bool NODE_OUT, int ACT>
static void wave_spmm_t(const seg_view& v, const void* vals, const void* Xt, int32_t B, void* Y,
                        float* carry, hipStream_t s) {
  const int32_t nblk = (int32_t)cdiv(v.S, WV_THREADS / SNK_WAVE);
  const int32_t xb =
      (PERM && nblk >= 8 * NUM_XCD) ? (int32_t)cdiv(nblk, NUM_XCD) : 0;
  const unsigned passes = (unsigned)cdiv(B, LPE * CH);
  const int32_t long_len = v.has_split ? v.tile : INT32_MAX;
  const int32_t sblk = xb ? xb * NUM_XCD : nblk;
  const int64_t x_elems = (int64_t)v.F * B;
  if (!v.has_split && passes == 1 &&
      wave_lds_fits(v, x_elems * (int64_t)sizeof(T), Xt, WL_MID_BYTES_SPMM, LPE)) {
    // two workgroups per CU (their LDS), or one per 16 segments if fewer
    const int32_t wl_blk = wave_lds_blocks(x_elems * (int64_t)sizeof(T), v.S);
    hipLaunchKernelGGL((k_wave_spmm_lds<T, CH, LPE, PERM, NODE_OUT, ACT>), dim3((unsigned)wl_blk),
                       dim3(WL_THREADS), (size_t)align_up((size_t)(x_elems * sizeof(T)), 16), s,
                       v.ptr, v.idx, v.perm, (const T*)vals, (const T*)Xt, (T*)Y, v.S, B,
                       x_elems);
    return;
  }
  if (!v.has_split) {
    hipLaunchKernelGGL((k_wave_spmm<T, CH, LPE, PERM, NODE_OUT, ACT>), dim3((unsigned)sblk, passes),
                       dim3(WV_THREADS), 0, s, v.ptr, v.idx, v.perm, (const T*)vals,
                       (const T*)Xt, (T*)Y, v.S, B, xb, long_len);
    return;
  }
  const int32_t pblk =
      (int32_t)(cdiv(cdiv(v.P, WV_THREADS / SNK_WAVE), NUM_XCD) * NUM_XCD);
  hipLaunchKernelGGL((k_wave_spmm_split<T, CH, LPE, PERM, NODE_OUT, ACT>),
                     dim3((unsigned)(pblk + sblk), passes), dim3(WV_THREADS), 0, s, v.ptr, v.idx,
                     v.perm, (const T*)vals, (const T*)Xt, (T*)Y, v.S, B, xb, long_len,
                     v.part_seg, v.part_nz, v.cut, carry, v.P, pblk);
  launch_fixup(v, sizeof(T) == 2 ? SNACK_BF16 : SNACK_F32, NODE_OUT, ACT, carry, Y, B, s);
}

template <typename T, int CH, int LPE>
static void wave_spmm_l(const seg_view& v, const void* vals, const void* Xt, int32_t B, void* Y,
                        bool node_out, int32_t act, float* carry, hipStream_t s) {
  if constexpr (CH * LPE <= 64) {
    const bool perm = v.perm != nullptr;
    if (perm) {
      if (node_out) wave_spmm_t<T, CH, LPE, true, true, ACT_NONE>(v, vals, Xt, B, Y, carry, s);
      else wave_spmm_t<T, CH, LPE, true, false, ACT_NONE>(v, vals, Xt, B, Y, carry, s);
    } else if (act == ACT_RELU) {
      if (node_out) wave_spmm_t<T, CH, LPE, false, true, ACT_RELU>(v, vals, Xt, B, Y, carry, s);
      else wave_spmm_t<T, CH, LPE, false, false, ACT_RELU>(v, vals, Xt, B, Y, carry, s);
    } else {
      if (node_out) wave_spmm_t<T, CH, LPE, false, true, ACT_NONE>(v, vals, Xt, B, Y, carry, s);
      else wave_spmm_t<T, CH, LPE, false, false, ACT_NONE>(v, vals, Xt, B, Y, carry, s);
    }
  }
}

template <typename T, int CH>
static void wave_spmm_c(const seg_view& v, const void* vals, const void* Xt, int32_t B, void* Y,
                        bool node_out, int32_t act, int lpe, float* carry, hipStream_t s) {
  switch (lpe) {
    case 1: wave_spmm_l<T, CH, 1>(v, vals, Xt, B, Y, node_out, act, carry, s); break;
    case 2: wave_spmm_l<T, CH, 2>(v, vals, Xt, B, Y, node_out, act, carry, s); break;
    case 4: wave_spmm_l<T, CH, 4>(v, vals, Xt, B, Y, node_out, act, carry, s); break;
    case 8: wave_spmm_l<T, CH, 8>(v, vals, Xt, B, Y, node_out, act, carry, s); break;
    default: wave_spmm_l<T, CH, 16>(v, vals, Xt, B, Y, node_out, act, carry, s); break;
  }
}

template <typename T>
static void wave_spmm_d(const seg_view& v, const void* vals, const void* Xt, int32_t B, void* Y,
                        bool node_out, int32_t act, const wave_shape& w, float* carry,
                        hipStream_t s) {
  switch (w.ch) {
    case 1: wave_spmm_c<T, 1>(v, vals, Xt, B, Y, node_out, act, w.lpe, carry, s); break;
    case 2: wave_spmm_c<T, 2>(v, vals, Xt, B, Y, node_out, act, w.lpe, carry, s); break;
    case 4: wave_spmm_c<T, 4>(v, vals, Xt, B, Y, node_out, act, w.lpe, carry, s); break;
    default:
      if constexpr (sizeof(T) == 2) wave_spmm_c<T, 8>(v, vals, Xt, B, Y, node_out, act, w.lpe, carry, s);
      break;
  }
}

template <typename T, int CH>
static bool wave_sddmm_c(const seg_view& v, const void* dYt, const void* Xt, int32_t B, void* dV,
                         int lpe, hipStream_t s) {
  const int32_t sblk = (int32_t)cdiv(v.S, WV_THREADS / SNK_WAVE);
  const int32_t pblk = (int32_t)cdiv(v.P, WV_THREADS / SNK_WAVE);
  const int32_t long_len = v.has_split ? v.tile : INT32_MAX;
  // X in LDS (see k_wave_spmm_lds): one batch pass, many rows, no split row
  const int64_t x_elems = (int64_t)v.F * B;
  const bool lds_ok =
      !v.has_split && wave_lds_fits(v, x_elems * (int64_t)sizeof(T), Xt, WL_MID_BYTES_SDDMM, lpe);
  const int32_t wl_blk = wave_lds_blocks(x_elems * (int64_t)sizeof(T), v.S);
  const size_t lds_bytes = align_up((size_t)(x_elems * sizeof(T)), 16);
#define SNK_WSD1(L, MULTI)                                                                      \
  do {                                                                                          \
    if (!v.has_split)                                                                           \
      hipLaunchKernelGGL((k_wave_sddmm<T, CH, L, MULTI>), dim3((unsigned)sblk),                 \
                         dim3(WV_THREADS), 0, s, v.ptr, v.idx, (const T*)dYt, (const T*)Xt,     \
                         (T*)dV, v.S, B, long_len);                                             \
    else                                                                                        \
      hipLaunchKernelGGL((k_wave_sddmm_split<T, CH, L, MULTI>), dim3((unsigned)(pblk + sblk)),  \
                         dim3(WV_THREADS), 0, s, v.ptr, v.idx, v.part_seg, v.part_nz, v.cut,    \
                         (const T*)dYt, (const T*)Xt, (T*)dV, v.S, v.P, B, long_len, pblk);     \
  } while (0)
#define SNK_WSD(L)                                                                       \
  do {                                                                                   \
    if (B > (L) * CH) {                                                                  \
      SNK_WSD1(L, true);                                                                 \
    } else if (lds_ok) {                                                                 \
      hipLaunchKernelGGL((k_wave_sddmm_lds<T, CH, L>), dim3((unsigned)wl_blk),           \
                         dim3(WL_THREADS), lds_bytes, s, v.ptr, v.idx, (const T*)dYt,    \
                         (const T*)Xt, (T*)dV, v.S, B, x_elems);                        \
    } else {                                                                             \
      SNK_WSD1(L, false);                                                                \
    }                                                                                    \
  } while (0)
  switch (lpe) {
    case 1: SNK_WSD(1); return true;
    case 2: SNK_WSD(2); return true;
    case 4: SNK_WSD(4); return true;
    case 8: SNK_WSD(8); return true;
    case 16: if constexpr (CH <= 4) { SNK_WSD(16); return true; } return false;
    default: return false;
  }
#undef SNK_WSD
#undef SNK_WSD1
}

}  // namespace snk
