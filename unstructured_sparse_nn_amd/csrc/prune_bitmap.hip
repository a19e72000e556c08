// prune_bitmap.hip -- prune/regrow over bitmaps of the M x K grid (gfx950).
//
// The rule is the one of snack_prune_regrow (drop the n_drop entries
// smallest in (|value| bits, row*K+col); grow the first n_drop positions of
// the SplitMix64 stream that lie outside the pre-step support and were not
// taken before; write survivors + grown back row-major).  This plan serves
// layers of density <= 1/4 whose support bitmap stays small; it needs no
// sort:
//   support  S, dropped D and grown G are bitmaps (bit b of word w is
//            position 32w + b).  Block b of the entry kernels owns the words
//            after the word of entry base_b - 1 up to the word of its last
//            entry, and writes each of them exactly once (zeros included),
//            so there is no fill kernel and no atomic;
//   select   radix select of the threshold magnitude, one 8-bit digit per
//            pass; each kernel picks the previous pass's digit itself from
//            the replicated histogram (a block scan), so no pick kernels;
//   regrow   stream indices are consumed in chunks whose size is the number
//            of positions still missing.  A chunk then cannot take more
//            than are missing, so taking every new distinct position of the
//            chunk (atomic test-and-set on G: order-free) gives exactly the
//            first n_drop acceptances of the stream.  The first chunks ride
//            on the select kernels (chunk 0 bucketed by grid region and
//            taken in LDS on grids up to 2^26 positions); one workgroup
//            finishes the tail;
//   write    new COO = the set bits of (S & ~D) | G in position order, a
//            survivor's value being the old value at its rank in S.
// One readback: the last kernel writes (error, positions missing) into the
// call's result words (the caller's pinned host words, or device words
// copied back); row/col/vals are written only on success.
#include <cmath>
#include <cstdlib>

#include "common.h"
#include "internal.h"
#include "results.h"
#include "prune_common.h"
#include "tiles.h"

namespace snk {
namespace {

constexpr int BT = 256;                   // threads per entry block
constexpr int BE = 4 * BT;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Streaming (non-temporal) store of four consecutive values.  The bitmap and
// value-copy writes of the entry kernels use these: measured, they shorten
// the drain before the next launch; the emitters' outputs, read soon after,
// measured slower with them.
template <typename T>
__device__ __forceinline__ void stream_store4(T* p, const vec<T, 4>& v) {
  if constexpr (sizeof(T) == 2) {
    u32x2 w;
    __builtin_memcpy(&w, &v, 8);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
  } else {
    u32x4 w;
    __builtin_memcpy(&w, &v, 16);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
  }
}
                // entries per block: thread t holds base + 4t .. + 3
constexpr int HREPL = 16;                 // select-histogram replicas
constexpr int AREPL = 64;                 // acceptance-count replicas
constexpr int SLOTS = 32;                 // grid-wide regrow chunks per call
constexpr int WT = 512;                   // threads (= bitmap words) per write block
// Entries per emitter block listed in LDS (one per thread per round): density
// up to 1/4 over a block of WT words; a denser block takes one thread per word.
constexpr int EMIT_CAP = 4096;
// Set bits per batch, their gathers in flight together, that a thread of the
// transposed-bitmap column emitter takes beyond its first few.
constexpr int EMIT_BATCH = 4;
constexpr int64_t PREFIX_INBLOCK_MAX = 4096;  // blocks up to which a block sums its own prefix
constexpr int FC_MAX_M = 12288;           // rows the column emitter stages in LDS
constexpr uint64_t AGG_FLAG = 1ull << 62;  // a published block count
constexpr int AGG_SPIN_MAX = 1 << 22;      // polls of one block count before giving up
constexpr int64_t STREAM_BOUND = 1ll << 40;
// Same-address device atomics serialise (~0.2 us each on gfx950), so blocks
// are fat (few blocks) and their counters spread over replicas.

struct bm_state {
  uint32_t pfx[4], msk[4];  // select: magnitude bits fixed after pass p
  int32_t need[4];          // drops still to place among entries matching pfx[p]
  int32_t err;              // 1 NaN, 2 index out of range, 4 COO order, 8 stream bound
  int32_t rem_final;        // positions still missing after the finisher
  int32_t pad[2];
  int64_t ch_start[SLOTS];  // chunk c: first stream index
  int32_t ch_rem[SLOTS];    // chunk c: positions missing at its start (= its length)
  int32_t ch_acc[SLOTS][AREPL];  // chunk c: positions it took, over AREPL counters
  int32_t hist[4][HREPL][256];   // select histograms; block b adds into replica b % HREPL
};

// FP in 16-row tiles: word (r, cw) of a K/32-word row at
// (r/16) * 16 K/32 + cw * 16 + r%16, so that a column word's words of 16
// consecutive rows fill one 128-byte line.
__host__ __device__ __forceinline__ int64_t fp_tile_index(int64_t r, int64_t cw, int64_t KW) {
  return (r >> 4) * (16 * KW) + cw * 16 + (r & 15);
}

__device__ __forceinline__ int32_t chunk_taken(const bm_state* st, int c) {
  int32_t a = 0;
#pragma unroll
  for (int i = 0; i < AREPL; ++i) a += st->ch_acc[c][i];
  return a;
}

__device__ __forceinline__ int64_t lin_of(int32_t r, int32_t c, int32_t M, int32_t K) {
  return (r < 0 || r >= M || c < 0 || c >= K) ? -1 : (int64_t)r * K + c;
}

// Exclusive block scans of NS values (ex, with block totals tot) and block
// sums of NR more, behind one barrier: each wave's scan totals and sums go
// through LDS together.  lds: NT/64 * (NS + NR) ints, left as written (the
// caller does not reuse it).  Call from all threads.
template <int NT, int NS, int NR>
__device__ __forceinline__ void block_scan_sum(const int32_t (&x)[NS], const int32_t (&y)[NR],
                                               int32_t* lds, int32_t (&ex)[NS],
                                               int32_t (&tot)[NS], int32_t (&sum)[NR]) {
  constexpr int NW = NT / SNK_WAVE, NV = NS + NR;
  const int w = threadIdx.x / SNK_WAVE;
  int32_t inc[NS], ys[NR];
#pragma unroll
  for (int k = 0; k < NS; ++k) inc[k] = wave_incl_scan_i32(x[k]);
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    ys[k] = y[k];
    for (int off = 32; off > 0; off >>= 1) ys[k] += __shfl_xor(ys[k], off, SNK_WAVE);
  }
  if (lane_id() == SNK_WAVE - 1) {
#pragma unroll
    for (int k = 0; k < NS; ++k) lds[w * NV + k] = inc[k];
#pragma unroll
    for (int k = 0; k < NR; ++k) lds[w * NV + NS + k] = ys[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    int32_t b = 0, t = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int32_t v = lds[i * NV + k];
      if (i < w) b += v;
      t += v;
    }
    ex[k] = b + inc[k] - x[k];
    tot[k] = t;
  }
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    int32_t t = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) t += lds[i * NV + NS + k];
    sum[k] = t;
  }
}

// Also zeroes zero[0 .. nzero) (the transposed bitmap's block sums of a fused
// prepare, which the transposer adds into).
__global__ __launch_bounds__(256) void k_bi_init(bm_state* st, int32_t* __restrict__ zero,
                                                 int64_t nzero) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < nzero) zero[i] = 0;
  if (i < 4 * HREPL * 256) (&st->hist[0][0][0])[i] = 0;
  if (i < SLOTS * AREPL) (&st->ch_acc[0][0])[i] = 0;
  if (i == 0) {
    st->err = 0;
    st->rem_final = 0;
  }
}

// Digit of select pass `pass` holding the need-th smallest remaining
// magnitude (one digit per thread, a block scan).  Output: the select state
// after the pass, which the block with `record` keeps for later kernels.
// 256 threads.
__device__ void pick_digit(bm_state* st, int pass, int shift, int32_t n_drop, uint32_t& pfx,
                          uint32_t& msk, int32_t& need, bool record) {
  __shared__ int32_t lds[BT / SNK_WAVE];
  __shared__ int32_t pick[2];
  const int t = threadIdx.x;
  const uint32_t p0 = pass ? st->pfx[pass - 1] : 0u;
  const uint32_t m0 = pass ? st->msk[pass - 1] : 0u;
  const int32_t n0 = pass ? st->need[pass - 1] : n_drop;
  int32_t h = 0;
#pragma unroll
  for (int r = 0; r < HREPL; ++r) h += st->hist[pass][r][t];
  int32_t tot;
  const int32_t ex = block_excl_scan_i32<BT>(h, lds, &tot);
  if (t == BT - 1) {  // guard: the last digit
    pick[0] = BT - 1;
    pick[1] = ex;
  }
  __syncthreads();
  if (ex < n0 && n0 <= ex + h) {
    pick[0] = t;
    pick[1] = ex;
  }
  __syncthreads();
  pfx = p0 | ((uint32_t)pick[0] << shift);
  msk = m0 | (255u << shift);
  need = n0 - pick[1];
  if (record && t == 0) {
    st->pfx[pass] = pfx;
    st->msk[pass] = msk;
    st->need[pass] = need;
  }
}

// Test-and-set candidates i0 + u*stride (u < 4, below `end`) on G unless
// they lie in S; all loads and atomics of the group are issued before any
// result is used.  Returns how many were taken.
__device__ __forceinline__ int32_t take_group(int64_t i0, int64_t stride, int64_t end,
                                              uint64_t stream, uint64_t MK,
                                              const uint32_t* __restrict__ sup,
                                              uint32_t* __restrict__ grown) {
  uint64_t p[4];
  uint32_t sw[4], old[4];
  bool ok[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = i0 + u * stride;
    ok[u] = i < end;
    p[u] = ok[u] ? sm64_position(stream, (uint64_t)i, MK) : 0;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) sw[u] = ok[u] ? sup[p[u] >> 5] : 0xFFFFFFFFu;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t bit = 1u << (p[u] & 31);
    old[u] = (sw[u] & bit) ? bit : atomicOr(&grown[p[u] >> 5], bit);
  }
  int32_t taken = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) taken += (old[u] & (1u << (p[u] & 31))) ? 0 : 1;
  return taken;
}

// Regrow chunk c (stream indices [start, start + rem), rem = positions still
// missing after chunk c-1), spread over the rbn workgroups that call it (rbi:
// this one's index among them).  A candidate is taken when it lies outside S
// and its bit in G was clear.  The kernels that carry a chunk give it
// workgroups of its own, so that its atomics (bound by the device's atomic
// throughput) overlap the kernel's other work.
__device__ void regrow_chunk(bm_state* st, int c, uint64_t stream, uint64_t MK, int32_t n_drop,
                             const uint32_t* __restrict__ sup, uint32_t* __restrict__ grown,
                             int64_t rbi, int64_t rbn) {
  __shared__ int32_t wsum[32];
  int64_t start = 0;
  int32_t rem = n_drop;
  if (c > 0) {
    start = st->ch_start[c - 1] + st->ch_rem[c - 1];
    rem = st->ch_rem[c - 1] - chunk_taken(st, c - 1);
  }
  if (rbi == 0 && threadIdx.x == 0) {
    st->ch_start[c] = start;
    st->ch_rem[c] = rem;
  }
  if (rem <= 0 || st->err) return;  // uniform over the grid
  if (start > STREAM_BOUND) {
    if (rbi == 0 && threadIdx.x == 0) atomicOr(&st->err, 8);
    return;
  }
  int32_t acc = 0;
  const int64_t end = start + rem;
  const int64_t stride = rbn * blockDim.x;
  for (int64_t i = start + rbi * blockDim.x + threadIdx.x; i < end; i += 4 * stride)
    acc += take_group(i, stride, end, stream, MK, sup, grown);
  // one atomic per block, spread over AREPL counters (same-address device
  // atomics serialise)
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, SNK_WAVE);
  if (lane_id() == 0) wsum[threadIdx.x / SNK_WAVE] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t b = 0;
    for (int i = 0; i < (int)(blockDim.x / SNK_WAVE); ++i) b += wsum[i];
    if (b) atomicAdd(&st->ch_acc[c][rbi % AREPL], b);
  }
}

// One workgroup (NT threads): chunks after grid chunk c-1 until nothing is
// missing (or the stream bound).  Records the positions still missing.
// (A first round over a window of draws deduplicated in an LDS hash and
// ranked in stream order by one block scan measured no faster: the window's
// draws, loads and probes cost as much as the rounds it saves.)
constexpr int FT = 1024;
constexpr int FINISH_ROUNDS = 4096;
template <int NT>
__device__ void regrow_tail(int32_t c, uint64_t stream, uint64_t MK, int32_t n_drop,
                            bm_state* st, const uint32_t* __restrict__ sup,
                            uint32_t* __restrict__ grown) {
  __shared__ int32_t red[NT / SNK_WAVE];
  const int t = threadIdx.x, nt = NT;
  int64_t start = 0;
  int32_t rem = n_drop;
  if (c > 0) {
    start = st->ch_start[c - 1] + st->ch_rem[c - 1];
    rem = st->ch_rem[c - 1] - chunk_taken(st, c - 1);
  }
  const bool ok = st->err == 0;
  // density <= 1/4 keeps the acceptance rate >= 1/2, so the remainder
  // roughly halves per round; the round cap only bounds a broken state
  for (int round = 0; ok && rem > 0; ++round) {
    if (start > STREAM_BOUND || round >= FINISH_ROUNDS) {
      if (t == 0) atomicOr(&st->err, 8);
      break;
    }
    int32_t acc = 0;
    for (int64_t i = start + t; i < start + rem; i += 4 * nt)
      acc += take_group(i, nt, start + rem, stream, MK, sup, grown);
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, SNK_WAVE);
    if (lane_id() == 0) red[t / SNK_WAVE] = acc;
    __syncthreads();
    int32_t taken = 0;
    for (int i = 0; i < nt / SNK_WAVE; ++i) taken += red[i];
    __syncthreads();
    start += rem;
    rem -= taken;
  }
  if (t == 0) st->rem_final = rem;
}

// Regrow chunk 0 without device atomics, for grids of up to 2^26 positions:
// the chunk's positions are bucketed by region (2^16 positions, 2,048
// bitmap words) by the bucketing workgroups (extra workgroups of the build
// kernel), and each region's workgroup (extra workgroups of the first
// select kernel) takes its candidates against S and an LDS copy of its G
// words, which it then stores whole.  Taking every new distinct position of
// the chunk is order-free, so the result is the same G as the atomic
// test-and-set over the grid.
constexpr int RB_SHIFT = 16;                      // positions per region: 2^16
constexpr int RB_WORDS = 1 << (RB_SHIFT - 5);     // bitmap words per region
constexpr int RB_PER = 8;                         // candidates per bucketing thread
constexpr int RB_CH = RB_PER * BT;                // stream indices per bucketing workgroup
constexpr int RB_MAXREG = 1024;                   // regions at most
constexpr int RB_MAXWG = 1024;                    // bucketing workgroups at most

// Bucketing workgroup j: stream indices [j*RB_CH, min(n_drop, (j+1)*RB_CH))
// of chunk 0 as positions, grouped by region into cand[j*RB_CH ..) (any
// order within a region), with tab[j*(nreg+1) + g] = the start of region
// g's group in that slice and tab[j*(nreg+1) + nreg] = the slice's count.
// BT threads.
__device__ void bucket_chunk0(int64_t j, uint64_t stream, uint64_t MK, int32_t n_drop,
                              int32_t nreg, uint32_t* __restrict__ cand,
                              int32_t* __restrict__ tab) {
  __shared__ int32_t h[RB_MAXREG];
  __shared__ int32_t lds[BT / SNK_WAVE];
  const int t = threadIdx.x;
  for (int g = t; g < nreg; g += BT) h[g] = 0;
  __syncthreads();
  const int64_t i0 = j * RB_CH;
  uint32_t p[RB_PER];
  int32_t rk[RB_PER];
#pragma unroll
  for (int u = 0; u < RB_PER; ++u) {
    const int64_t i = i0 + u * BT + t;
    p[u] = i < n_drop ? (uint32_t)sm64_position(stream, (uint64_t)i, MK) : 0u;
  }
#pragma unroll
  for (int u = 0; u < RB_PER; ++u)
    rk[u] = i0 + u * BT + t < n_drop ? atomicAdd(&h[p[u] >> RB_SHIFT], 1) : -1;
  __syncthreads();
  constexpr int GPT = RB_MAXREG / BT;  // regions per thread in the scan
  int32_t v[GPT], sum = 0;
#pragma unroll
  for (int k = 0; k < GPT; ++k) {
    const int g = t * GPT + k;
    v[k] = g < nreg ? h[g] : 0;
    sum += v[k];
  }
  int32_t tot;
  int32_t ex = block_excl_scan_i32<BT>(sum, lds, &tot);  // its barriers order the reads of h
  int32_t* row_tab = tab + j * (nreg + 1);
#pragma unroll
  for (int k = 0; k < GPT; ++k) {
    const int g = t * GPT + k;
    if (g < nreg) {
      h[g] = ex;
      row_tab[g] = ex;
    }
    ex += v[k];
  }
  if (t == 0) row_tab[nreg] = tot;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < RB_PER; ++u)
    if (rk[u] >= 0) cand[i0 + h[p[u] >> RB_SHIFT] + rk[u]] = p[u];
}

// Region g's workgroup of chunk 0 (BT threads): its candidates from the nwg
// bucketing slices, each taken if outside S and new in G (an LDS
// test-and-set); the region's G words are stored whole (zeros included) and
// the count taken is added into chunk 0's acceptance counters.
__device__ void region_chunk0(int32_t g, bm_state* st, int32_t n_drop, int32_t nreg,
                              int32_t nwg, int64_t W, const uint32_t* __restrict__ cand,
                              const int32_t* __restrict__ tab, const uint32_t* __restrict__ sup,
                              uint32_t* __restrict__ grown) {
  __shared__ uint32_t Ss[RB_WORDS], Gs[RB_WORDS];
  __shared__ int32_t run0[RB_MAXWG], start[RB_MAXWG];
  __shared__ int32_t lds[BT / SNK_WAVE];
  const int t = threadIdx.x;
  const int64_t wbase = (int64_t)g * RB_WORDS;
  // the region's S words and the slice table, every load in flight at once
  // (indices clamped in range, unused values discarded afterwards)
  constexpr int SPT = RB_WORDS / BT;   // S words per thread
  constexpr int WPTH = RB_MAXWG / BT;  // slices per thread in the scan
  uint32_t sw[SPT];
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const int64_t w = wbase + k * BT + t;
    sw[k] = sup[w < W ? w : W - 1];
  }
  // slice table: with slices of >= 2 threads, the thread's own slice's run
  // bounds in a[0], a[1]; else WPTH slices per thread for the scan below
  int32_t a[WPTH], len[WPTH], sum = 0;
  if (2 * nwg <= BT) {
    const int sl = t / (BT / nwg);
    const int64_t ti = (int64_t)(sl < nwg ? sl : nwg - 1) * (nreg + 1) + g;
    a[0] = tab[ti];
    a[1] = tab[ti + 1];
  } else {
#pragma unroll
    for (int k = 0; k < WPTH; ++k) {
      const int wgi = t * WPTH + k;
      const int64_t ti = (int64_t)(wgi < nwg ? wgi : nwg - 1) * (nreg + 1) + g;
      a[k] = tab[ti];
      len[k] = tab[ti + 1];
    }
  }
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    Ss[k * BT + t] = wbase + k * BT + t < W ? sw[k] : 0xFFFFFFFFu;
    Gs[k * BT + t] = 0u;
  }
  int32_t taken = 0;
  // take candidate pc (a region position) if outside S and new in G
  auto take = [&](uint32_t pc) {
    const uint32_t loc = pc & ((1u << RB_SHIFT) - 1u);
    const uint32_t bit = 1u << (loc & 31);
    if (Ss[loc >> 5] & bit) return;
    if (!(atomicOr(&Gs[loc >> 5], bit) & bit)) ++taken;
  };
  if (2 * nwg <= BT) {  // block-uniform: each slice's run split over tps threads
    const int tps = BT / nwg;
    const int sl = t / tps, sub = t - sl * tps;
    const bool mine = sl < nwg;
    const int32_t ln = mine ? a[1] - a[0] : 0;  // (a[0], a[1]): the slice's run bounds
    const int64_t cb = (int64_t)(mine ? sl : 0) * RB_CH + a[0];
    // the first candidates' loads go out before the barrier that publishes
    // Ss and Gs (an unused slot reads element 0, L1-resident; discarded)
    uint32_t pc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int32_t i = sub + u * tps;
      pc[u] = cand[i < ln ? cb + i : 0];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (sub + u * tps < ln) take(pc[u]);
    for (int32_t i0 = sub + 4 * tps; i0 < ln; i0 += 4 * tps) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int32_t i = i0 + u * tps;
        pc[u] = cand[i < ln ? cb + i : 0];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i0 + u * tps < ln) take(pc[u]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < WPTH; ++k) {
      const bool in = t * WPTH + k < nwg;
      len[k] = in ? len[k] - a[k] : 0;
      a[k] = in ? a[k] : 0;
      sum += len[k];
    }
    int32_t n_g;
    int32_t ex = block_excl_scan_i32<BT>(sum, lds, &n_g);
#pragma unroll
    for (int k = 0; k < WPTH; ++k) {
      const int wgi = t * WPTH + k;
      if (wgi < nwg) {
        run0[wgi] = ex;
        start[wgi] = wgi * RB_CH + a[k];
      }
      ex += len[k];
    }
    __syncthreads();
    int top = 1;  // the largest power of two below nwg (1 if nwg <= 2)
    while (2 * top < nwg) top *= 2;
    for (int32_t b0 = 0; b0 < n_g; b0 += 4 * BT) {
      uint32_t pc[4];
      bool ok[4];
      int32_t e[4], lo[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        e[u] = b0 + u * BT + t;
        ok[u] = e[u] < n_g;
        lo[u] = 0;  // run0[0] = 0 <= e
      }
      // the last slice whose run starts at or before e: a branch-free search
      // with the four candidates' LDS reads of each step in flight together
      for (int step = top; step > 0; step >>= 1) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int m = lo[u] + step;
          if (m < nwg && run0[m] <= e[u]) lo[u] = m;
        }
      }
      // an unused slot reads the first element (L1-resident; discarded)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        pc[u] = cand[ok[u] ? start[lo[u]] + (e[u] - run0[lo[u]]) : 0];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (ok[u]) take(pc[u]);
    }
  }
  __syncthreads();
  for (int k = t; k < RB_WORDS; k += BT) {
    const int64_t w = wbase + k;
    if (w < W) grown[w] = Gs[k];
  }
  int32_t tot;
  block_excl_scan_i32<BT>(taken, lds, &tot);
  if (t == 0) {
    if (tot) atomicAdd(&st->ch_acc[0][g % AREPL], tot);
    if (g == 0) {
      st->ch_start[0] = 0;
      st->ch_rem[0] = n_drop;
    }
  }
}

// The entries a block needs beyond its own, loaded by every thread next to
// the block's main loads (clamped indices, no branch, one round trip) and
// kept by a few threads in LDS: the linear index of entry base-1 (-1 for
// block 0 or an invalid entry) and of the next NEXT entries past the block
// (-1 past nnz or invalid), with their magnitudes if mag is given.  A
// bitmap word holds 32 positions, so at most 32 later entries can share the
// block's last word.  edge_load issues the loads; edge_store, called once
// the caller's other loads are out, fills LDS; readers wait for the
// block's next barrier.
constexpr int NEXT = 32;
template <typename T>
struct edge_vals {
  int32_t er, ec, nr, nc;
  T nv;
};
template <typename T>
__device__ __forceinline__ edge_vals<T> edge_load(const int32_t* __restrict__ row,
                                                  const int32_t* __restrict__ col,
                                                  const T* __restrict__ vals, int64_t nnz,
                                                  int64_t base, int n) {
  const int64_t eb = base > 0 ? base - 1 : 0;
  const int64_t k = base + n + (threadIdx.x & (NEXT - 1));
  const int64_t kk = k < nnz ? k : nnz - 1;
  return edge_vals<T>{row[eb], col[eb], row[kk], col[kk], vals[kk]};
}
template <typename T>
__device__ __forceinline__ void edge_store(const edge_vals<T>& e, int64_t nnz, int32_t M,
                                           int32_t K, int64_t base, int n, int64_t* edge,
                                           int64_t* nxt, uint32_t* mag) {
  const int t = threadIdx.x;
  const int64_t k = base + n + (t & (NEXT - 1));
  if (t == BT - 1) *edge = base > 0 ? lin_of(e.er, e.ec, M, K) : -1;
  if (t < NEXT) {
    nxt[t] = k < nnz ? lin_of(e.nr, e.nc, M, K) : -1;
    if (mag) mag[t] = magnitude<T>(raw_bits(e.nv));
  }
}

// Bitmap words [w_lo, w_hi] of an entry block, written whole (zeros
// included) with coalesced stores.  Each chunk of up to CAP words is
// assembled in LDS -- an LDS atomicOr per flagged entry (l[q] >= 0,
// f[q]) of the calling thread whose word lies in the chunk, plus `extra`
// into word w_hi -- and then stored; b, if given, receives zeros over the
// same words.  An entry whose word lies outside the range (a block's first
// run, in the previous block's last word) is left to that word's owner.
// w_lo, w_hi and extra's presence are block-uniform; call from all threads.
constexpr int CAP = 2048;
__device__ void write_block_words(uint32_t* buf, int64_t w_lo, int64_t w_hi,
                                  const int64_t (&l)[4], const bool (&f)[4], uint32_t extra,
                                  uint32_t* __restrict__ a, uint32_t* __restrict__ b) {
  for (int64_t cs = w_lo; cs <= w_hi; cs += CAP) {
    const int32_t len = (int32_t)std::min<int64_t>(CAP, w_hi + 1 - cs);
    for (int j = threadIdx.x; j < len; j += BT) buf[j] = 0u;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t w = l[q] >> 5;
      if (f[q] && l[q] >= 0 && w >= cs && w < cs + len)
        atomicOr(&buf[w - cs], 1u << (l[q] & 31));
    }
    if (threadIdx.x == 0 && extra && w_hi < cs + len) atomicOr(&buf[w_hi - cs], extra);
    __syncthreads();
    for (int j = threadIdx.x; j < len; j += BT) {
      __builtin_nontemporal_store(buf[j], &a[cs + j]);
      if (b) __builtin_nontemporal_store(0u, &b[cs + j]);
    }
    __syncthreads();
  }
}

// Word of a block's last entry (entry n-1, held by thread (n-1)/4), into
// *whi (-1 if that entry is invalid).
__device__ __forceinline__ void last_word(const int64_t (&l)[4], int n, int64_t* whi) {
  const int t = threadIdx.x, i = n - 1;
  if (t == (i >> 2)) {
    const int q = i & 3;
    const int64_t x = q == 0 ? l[0] : q == 1 ? l[1] : q == 2 ? l[2] : l[3];
    *whi = x < 0 ? -1 : (x >> 5);
  }
}

// Support bitmap S (and G cleared, unless chunk 0 is bucketed: grown is
// then NULL), a copy of the values, the NaN / index / order checks and the
// first select histogram.  Thread t holds entries base + 4t .. base + 4t + 3.
// The first gridDim.x - nblk workgroups bucket regrow chunk 0 (bucket_chunk0):
// the regrow is the longer chain, so its workgroups are dispatched first.
template <typename T>
__global__ __launch_bounds__(BT) void k_bi_build(
    const int32_t* __restrict__ row, const int32_t* __restrict__ col, const T* __restrict__ vals,
    int64_t nnz, int32_t M, int32_t K, int64_t W, int shift, int32_t vec_ok, bm_state* st,
    uint32_t* __restrict__ sup, uint32_t* __restrict__ grown, T* __restrict__ vals_ws,
    int64_t nblk, uint64_t stream, uint64_t MK, int32_t n_drop, int32_t nreg,
    uint32_t* __restrict__ cand, int32_t* __restrict__ tab) {
  const int64_t nx = (int64_t)gridDim.x - nblk;
  if ((int64_t)blockIdx.x < nx) {  // bucketing workgroups of regrow chunk 0
    bucket_chunk0((int64_t)blockIdx.x, stream, MK, n_drop, nreg, cand, tab);
    return;
  }
  const int64_t bid = (int64_t)blockIdx.x - nx;
  __shared__ int32_t h[256];
  __shared__ uint32_t buf[CAP];
  __shared__ int64_t lastl[BT];
  __shared__ int64_t edge_s, whi_s;
  __shared__ int64_t nxt[NEXT];
  const int t = threadIdx.x;
  h[t] = 0;
  const int64_t base = bid * BE;
  const int n = (int)std::min<int64_t>(BE, nnz - base);
  const int64_t k0 = base + 4 * t;
  const bool full = vec_ok && k0 + 3 < nnz;
  int32_t r4[4], c4[4];
  T v4[4];
  if (full) {
    const int4 rv = *reinterpret_cast<const int4*>(row + k0);
    const int4 cv = *reinterpret_cast<const int4*>(col + k0);
    const vec<T, 4> vv = *reinterpret_cast<const vec<T, 4>*>(vals + k0);
    r4[0] = rv.x; r4[1] = rv.y; r4[2] = rv.z; r4[3] = rv.w;
    c4[0] = cv.x; c4[1] = cv.y; c4[2] = cv.z; c4[3] = cv.w;
#pragma unroll
    for (int j = 0; j < 4; ++j) v4[j] = vv.v[j];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = k0 + j < nnz;
      r4[j] = ok ? row[k0 + j] : 0;
      c4[j] = ok ? col[k0 + j] : 0;
      v4[j] = ok ? vals[k0 + j] : (T)0;
    }
  }
  const edge_vals<T> ev = edge_load<T>(row, col, vals, nnz, base, n);
  edge_store<T>(ev, nnz, M, K, base, n, &edge_s, nxt, nullptr);
  __syncthreads();  // h zeroed before any wave adds to it
  int err = 0;
  int64_t l[4];
  bool f[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool ok = k0 + j < nnz;
    const uint32_t a = magnitude<T>(raw_bits(v4[j]));
    wave_hist_add(h, (a >> shift) & 255u, ok);
    l[j] = ok ? lin_of(r4[j], c4[j], M, K) : -1;
    f[j] = ok;
    if (ok && is_nan_mag<T>(a)) err |= 1;
    if (ok && l[j] < 0) err |= 2;
  }
  if (full) {
    vec<T, 4> vv;
#pragma unroll
    for (int j = 0; j < 4; ++j) vv.v[j] = v4[j];
    stream_store4(vals_ws + k0, vv);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (k0 + j < nnz) vals_ws[k0 + j] = v4[j];
  }
  lastl[t] = l[3];
  last_word(l, n, &whi_s);
  __syncthreads();
  // strictly increasing: against the previous entry (the block's left edge
  // staged in LDS)
  const int64_t edge = edge_s;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (l[q] < 0) continue;
    const int64_t pl = q > 0 ? l[q - 1] : (t > 0 ? lastl[t - 1] : edge);
    if (pl >= 0 && l[q] <= pl) err |= 4;
  }
  const bool last_block = base + n >= nnz;
  const int64_t w_lo = edge >= 0 ? (edge >> 5) + 1 : 0;
  const int64_t w_hi = last_block ? W - 1 : whi_s;
  uint32_t extra = 0;
  if (t == 0 && !last_block) {  // next block's entries in this block's last word
    for (int u = 0; u < NEXT; ++u) {
      const int64_t x = nxt[u];
      if (x < 0 || (x >> 5) != w_hi) break;
      extra |= 1u << (x & 31);
    }
  }
  write_block_words(buf, w_lo, w_hi, l, f, extra, sup, grown);
  if (err) atomicOr(&st->err, err);
  if (h[t]) atomicAdd(&st->hist[0][bid % HREPL][t], h[t]);
}

// Select pass `pass` >= 1: pick the previous pass's digit, histogram the
// next digit of the entries matching the prefix.  The first gridDim.x - nblk
// workgroups run regrow chunk c (with nwg > 0: chunk 0 by region,
// region_chunk0).
template <typename T>
__global__ __launch_bounds__(BT) void k_bi_sel(const T* __restrict__ vals, int64_t nnz,
                                               int64_t nblk, int pass, int prev_shift, int shift,
                                               int32_t n_drop, int32_t c, uint64_t stream,
                                               uint64_t MK, bm_state* st,
                                               const uint32_t* __restrict__ sup,
                                               uint32_t* __restrict__ grown, int32_t nreg,
                                               int32_t nwg, int64_t W,
                                               const uint32_t* __restrict__ cand,
                                               const int32_t* __restrict__ tab) {
  __shared__ int32_t h[256];
  const int64_t nx = (int64_t)gridDim.x - nblk;
  if ((int64_t)blockIdx.x < nx) {
    if (nwg > 0)  // chunk 0 from the buckets, one workgroup per region
      region_chunk0((int32_t)blockIdx.x, st, n_drop, nreg, nwg, W, cand, tab, sup, grown);
    else
      regrow_chunk(st, c, stream, MK, n_drop, sup, grown, blockIdx.x, nx);
    return;
  }
  const int64_t bid = (int64_t)blockIdx.x - nx;
  const int t = threadIdx.x;
  h[t] = 0;
  const int64_t k0 = bid * BE + 4 * t;
  uint32_t a[4];
  T x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = vals[k0 + j < nnz ? k0 + j : nnz - 1];  // loads in flight together
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = k0 + j < nnz ? magnitude<T>(raw_bits(x[j])) : 0u;
  uint32_t pfx, msk;
  int32_t need;
  pick_digit(st, pass - 1, prev_shift, n_drop, pfx, msk, need, bid == 0);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    wave_hist_add(h, (a[j] >> shift) & 255u, k0 + j < nnz && (a[j] & msk) == pfx);
  __syncthreads();
  if (h[t]) atomicAdd(&st->hist[pass][bid % HREPL][t], h[t]);
}

// Last pick (the threshold magnitude tau and the ties to drop), entries at
// tau per block.  The first gridDim.x - nblk workgroups run regrow chunk c.
template <typename T>
__global__ __launch_bounds__(BT) void k_bi_count(const T* __restrict__ vals, int64_t nnz,
                                                 int64_t nblk, int last_pass, int shift,
                                                 int32_t n_drop, int32_t c, uint64_t stream,
                                                 uint64_t MK, bm_state* st,
                                                 int32_t* __restrict__ cnt_eq,
                                                 const uint32_t* __restrict__ sup,
                                                 uint32_t* __restrict__ grown) {
  __shared__ int32_t lds[BT / SNK_WAVE];
  const int64_t nx = (int64_t)gridDim.x - nblk;
  if ((int64_t)blockIdx.x < nx) {
    regrow_chunk(st, c, stream, MK, n_drop, sup, grown, blockIdx.x, nx);
    return;
  }
  const int64_t bid = (int64_t)blockIdx.x - nx;
  const int64_t k0 = bid * BE + 4 * threadIdx.x;
  uint32_t a[4];
  T x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = vals[k0 + j < nnz ? k0 + j : nnz - 1];  // loads in flight together
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = k0 + j < nnz ? magnitude<T>(raw_bits(x[j])) : 0xFFFFFFFFu;
  uint32_t tau, msk;
  int32_t need;
  pick_digit(st, last_pass, shift, n_drop, tau, msk, need, bid == 0);
  int32_t eq = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) eq += a[j] == tau ? 1 : 0;
  int32_t tot;
  block_excl_scan_i32<BT>(eq, lds, &tot);
  if (threadIdx.x == 0) cnt_eq[bid] = tot;
}

// One workgroup: base_eq[b] = entries at tau in blocks before b (used when
// there are too many blocks for each to sum its own prefix).
__global__ __launch_bounds__(1024) void k_bi_eq_scan(const int32_t* __restrict__ cnt_eq,
                                                     int32_t* __restrict__ base_eq, int64_t nblk) {
  __shared__ int32_t lds[1024 / SNK_WAVE];
  int32_t run = 0;
  for (int64_t c = 0; c < nblk; c += 1024) {
    const int64_t b = c + threadIdx.x;
    const int32_t v = b < nblk ? cnt_eq[b] : 0;
    int32_t tot;
    const int32_t ex = block_excl_scan_i32<1024>(v, lds, &tot);
    if (b < nblk) base_eq[b] = run + ex;
    run += tot;
  }
}


// Dropped bitmap D: entry k is dropped if its magnitude is below tau, or at
// tau with tie rank (index order) below need.  The first gridDim.x - nblk
// workgroups run regrow chunk c; with `tail` a single one runs chunk c and
// all the rest.
template <typename T>
__global__ __launch_bounds__(BT) void k_bi_drop(
    const int32_t* __restrict__ row, const int32_t* __restrict__ col, const T* __restrict__ vals,
    int64_t nnz, int64_t nblk, int32_t M, int32_t K, int64_t W, int last_pass,
    const int32_t* __restrict__ cnt_eq,
    const int32_t* __restrict__ base_eq, int32_t n_drop, int32_t c, uint64_t stream, uint64_t MK,
    bm_state* st, uint32_t* __restrict__ dropb, const uint32_t* __restrict__ sup,
    uint32_t* __restrict__ grown, int32_t tail) {
  __shared__ int32_t lds[BT / SNK_WAVE * 2];
  __shared__ uint32_t buf[CAP];
  __shared__ int64_t edge_s, whi_s;
  __shared__ int64_t nxt[NEXT];
  __shared__ uint32_t nxt_mag[NEXT];
  const int64_t nx = (int64_t)gridDim.x - nblk;
  if ((int64_t)blockIdx.x < nx) {
    if (tail)  // one workgroup: chunk c and every later one (no finisher launch)
      regrow_tail<BT>(c, stream, MK, n_drop, st, sup, grown);
    else
      regrow_chunk(st, c, stream, MK, n_drop, sup, grown, blockIdx.x, nx);
    return;
  }
  const int64_t bid = (int64_t)blockIdx.x - nx;
  const int t = threadIdx.x;
  const int64_t base = bid * BE;
  const int n = (int)std::min<int64_t>(BE, nnz - base);
  const int64_t k0 = base + 4 * t;
  // every load first (clamped indices): the block's entries, its edge
  // entries, its share of the tie counts of earlier blocks (four per thread
  // here) and the threshold state
  int32_t r4[4], c4[4];
  T v4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t kk = k0 + j < nnz ? k0 + j : nnz - 1;
    v4[j] = vals[kk];
    r4[j] = row[kk];
    c4[j] = col[kk];
  }
  const edge_vals<T> ev = edge_load<T>(row, col, vals, nnz, base, n);
  int32_t pe[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = t + (int64_t)u * BT;
    pe[u] = base_eq ? 0 : cnt_eq[i < bid ? i : 0];
  }
  const int32_t e_pre = base_eq ? base_eq[bid] : 0;
  const uint32_t tau = st->pfx[last_pass];
  const int32_t need = st->need[last_pass];
  uint32_t a[4];
  int64_t l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool ok = k0 + j < nnz;
    a[j] = ok ? magnitude<T>(raw_bits(v4[j])) : 0xFFFFFFFFu;
    l[j] = ok ? lin_of(r4[j], c4[j], M, K) : -1;
  }
  edge_store<T>(ev, nnz, M, K, base, n, &edge_s, nxt, nxt_mag);
  last_word(l, n, &whi_s);
  int32_t part = 0;
  if (!base_eq) {
#pragma unroll
    for (int u = 0; u < 4; ++u) part += t + (int64_t)u * BT < bid ? pe[u] : 0;
    for (int64_t i = t + 4 * (int64_t)BT; i < bid; i += BT) part += cnt_eq[i];
  }
  // tie ranks in index order and the entries at tau before the block, in
  // one block scan (its barrier also publishes the staged edges)
  int32_t eq = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) eq += a[j] == tau ? 1 : 0;
  int32_t ex1[1], tt1[1], sm1[1];
  {
    const int32_t xs[1] = {eq};
    const int32_t ys[1] = {part};
    block_scan_sum<BT, 1, 1>(xs, ys, lds, ex1, tt1, sm1);
  }
  const int32_t E = base_eq ? e_pre : sm1[0];
  const int32_t tot = tt1[0];
  int32_t er = E + ex1[0];
  const int32_t run = E + tot;
  bool f[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool is_eq = a[j] == tau;
    f[j] = l[j] >= 0 && (a[j] < tau || (is_eq && er < need));
    er += is_eq ? 1 : 0;
  }
  const int64_t edge = edge_s;
  const bool last_block = base + n >= nnz;
  const int64_t w_lo = edge >= 0 ? (edge >> 5) + 1 : 0;
  const int64_t w_hi = last_block ? W - 1 : whi_s;
  uint32_t extra = 0;
  if (t == 0 && !last_block) {  // next block's entries in this word, with their tie ranks
    int32_t ern = run;
    for (int u = 0; u < NEXT; ++u) {
      const int64_t x = nxt[u];
      if (x < 0 || (x >> 5) != w_hi) break;
      const uint32_t m = nxt_mag[u];
      if (m < tau || (m == tau && ern < need)) extra |= 1u << (x & 31);
      ern += m == tau ? 1 : 0;
    }
  }
  write_block_words(buf, w_lo, w_hi, l, f, extra, dropb, nullptr);
}

// A regrow chunk on its own (only when the acceptance rate is low).
__global__ __launch_bounds__(BT) void k_bi_chunk(int32_t c, uint64_t stream, uint64_t MK,
                                                 int32_t n_drop, bm_state* st,
                                                 const uint32_t* __restrict__ sup,
                                                 uint32_t* __restrict__ grown) {
  regrow_chunk(st, c, stream, MK, n_drop, sup, grown, blockIdx.x, gridDim.x);
}

__global__ __launch_bounds__(FT) void k_bi_finish(int32_t c, uint64_t stream, uint64_t MK,
                                                  int32_t n_drop, bm_state* st,
                                                  const uint32_t* __restrict__ sup,
                                                  uint32_t* __restrict__ grown) {
  regrow_tail<FT>(c, stream, MK, n_drop, st, sup, grown);
}

__device__ __forceinline__ int4 word_counts(uint32_t S, uint32_t D, uint32_t G) {
  return make_int4(__popc((S & ~D) | G), __popc(S), __popc(D), __popc(G));
}

__device__ __forceinline__ int4 add4(int4 a, int4 b) {
  return make_int4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// Per block of WT words: popcounts of (new support, old support, dropped,
// grown).
__global__ __launch_bounds__(WT) void k_bi_wsum(const uint32_t* __restrict__ sup,
                                                const uint32_t* __restrict__ dropb,
                                                const uint32_t* __restrict__ grown, int64_t W,
                                                int4* __restrict__ bsum) {
  __shared__ int4 lds[WT / SNK_WAVE];
  const int64_t w = (int64_t)blockIdx.x * WT + threadIdx.x;
  int4 c = w < W ? word_counts(sup[w], dropb[w], grown[w]) : make_int4(0, 0, 0, 0);
  for (int off = 32; off > 0; off >>= 1) {
    c.x += __shfl_xor(c.x, off, SNK_WAVE);
    c.y += __shfl_xor(c.y, off, SNK_WAVE);
    c.z += __shfl_xor(c.z, off, SNK_WAVE);
    c.w += __shfl_xor(c.w, off, SNK_WAVE);
  }
  if (lane_id() == 0) lds[threadIdx.x / SNK_WAVE] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int4 tot = make_int4(0, 0, 0, 0);
    for (int i = 0; i < WT / SNK_WAVE; ++i) tot = add4(tot, lds[i]);
    bsum[blockIdx.x] = tot;
  }
}

// One workgroup: exclusive prefix of n int4 block sums (thread t owns a
// contiguous segment).  Only used for very large bitmaps.
__global__ __launch_bounds__(1024) void k_bi_bscan(const int4* __restrict__ in,
                                                   int4* __restrict__ out, int64_t n) {
  __shared__ int32_t lds[1024 / SNK_WAVE];
  const int64_t per = cdiv_dev(n, 1024);
  const int64_t a = std::min<int64_t>(n, (int64_t)threadIdx.x * per);
  const int64_t b = std::min<int64_t>(n, a + per);
  int4 s = make_int4(0, 0, 0, 0);
  for (int64_t i = a; i < b; ++i) s = add4(s, in[i]);
  int32_t tot;
  int4 e;
  e.x = block_excl_scan_i32<1024>(s.x, lds, &tot);
  e.y = block_excl_scan_i32<1024>(s.y, lds, &tot);
  e.z = block_excl_scan_i32<1024>(s.z, lds, &tot);
  e.w = block_excl_scan_i32<1024>(s.w, lds, &tot);
  for (int64_t i = a; i < b; ++i) {
    out[i] = e;
    e = add4(e, in[i]);
  }
}

// New COO (the set bits of (S & ~D) | G in position order), the dropped and
// grown lists, and optionally the new support F and its per-word exclusive
// prefix counts; one thread per bitmap word.  Block 0 reports (error,
// positions missing) into pinned host memory; nothing else is written
// unless both are 0.  Writes are clamped to nnz / n_drop.
template <typename T, bool LISTS>
__global__ __launch_bounds__(WT, LISTS ? 5 : 8) void k_bi_emit(
    const uint32_t* __restrict__ sup, const uint32_t* __restrict__ dropb,
    const uint32_t* __restrict__ grown, int64_t W, const int4* __restrict__ bsum,
    const int4* __restrict__ boff, const T* __restrict__ vals_ws, int32_t K, int32_t small_grid,
    int64_t nnz, int64_t n_drop, const bm_state* st, int32_t* __restrict__ result,
    uint2* __restrict__ FP, int32_t fp_tiled, int32_t* __restrict__ rs_blk,
    uint64_t* __restrict__ agg, int32_t* __restrict__ row,
    int32_t* __restrict__ col, T* __restrict__ vals, int64_t* __restrict__ dropped_lin,
    int64_t* __restrict__ grown_lin) {
  __shared__ int32_t lds[WT / SNK_WAVE * 7];
  __shared__ int32_t red2[WT / SNK_WAVE][2];
  __shared__ uint32_t ent[EMIT_CAP];  // (word in block << 5) | bit, in output order
  __shared__ uint32_t sS[WT];
  __shared__ int32_t sq[WT], sr[WT], sc[WT];
  const int t = threadIdx.x;
  // every load that depends on nothing is issued first: the block's words,
  // the block sums before it (up to 2 WT of them here) and the state words
  const int64_t w = (int64_t)blockIdx.x * WT + t;
  const int64_t wc = w < W ? w : W - 1;
  const uint32_t S0 = sup[wc], D0 = dropb[wc], G0 = grown[wc];
  const int64_t nb_before = (int64_t)blockIdx.x;
  // (without the dropped and grown lists only the first two block counts
  // are needed)
  int4 p0 = make_int4(0, 0, 0, 0), p1 = make_int4(0, 0, 0, 0);
  if (!boff && !agg && nb_before > 0) {
    if constexpr (LISTS) {
      p0 = bsum[t < nb_before ? t : 0];
      p1 = bsum[t + WT < nb_before ? t + WT : 0];
    } else {
      const int2 a = *reinterpret_cast<const int2*>(&bsum[t < nb_before ? t : 0]);
      const int2 b = *reinterpret_cast<const int2*>(&bsum[t + WT < nb_before ? t + WT : 0]);
      p0 = make_int4(a.x, a.y, 0, 0);
      p1 = make_int4(b.x, b.y, 0, 0);
    }
  }
  const int32_t err = st->err, missing = st->rem_final;
  if (blockIdx.x == 0 && t == 0) {
    store_result(&result[0], err);
    store_result(&result[1], missing);
    store_result(&result[2], 0);  // split flags of a fused prepare, set by later kernels
    store_result(&result[3], 0);
  }
  if (err || missing > 0) return;
  // this thread's share of the block base (the sum of the sums of earlier
  // blocks); the block reduces it with the two scans below
  int4 part = make_int4(0, 0, 0, 0);
  if (!boff && !agg) {
    if (t < nb_before) part = p0;
    if (t + WT < nb_before) part = add4(part, p1);
    for (int64_t i = t + 2 * WT; i < nb_before; i += 2 * WT) {  // two loads in flight
      const int64_t i2 = i + WT < nb_before ? i + WT : i;
      const int4 x = bsum[i], y = bsum[i2];
      part = add4(part, i2 != i ? add4(x, y) : x);
    }
  }
  const uint32_t S = w < W ? S0 : 0u, D = w < W ? D0 : 0u, G = w < W ? G0 : 0u;
  const int4 c = word_counts(S, D, G);
  const uint32_t F0 = (S & ~D) | G;
  const int64_t pw = w * 32;
  // row and column of the word's first position; the rest step from it
  int32_t r0 = 0, c0 = 0;
  if (F0 || fp_tiled) {
    if (small_grid) {
      r0 = (int32_t)((uint32_t)pw / (uint32_t)K);
      c0 = (int32_t)((uint32_t)pw - (uint32_t)r0 * (uint32_t)K);
    } else {
      r0 = (int32_t)(pw / K);
      c0 = (int32_t)(pw - (int64_t)r0 * K);
    }
  }
  // for the column emitter: the sum over rows of the new row starts equals
  // sum_r count(r) * (M - 1 - r); each block adds its words' terms
  const int32_t rsw = fp_tiled && w < W ? c.x * (int32_t)(W / (K >> 5) - 1 - r0) : 0;
  // a block holds at most 32 * WT = 16384 positions, so two counts share an
  // int32 (15 bits each, no overflow): two scans serve all four
  int32_t fs, nf, dg = 0, rs_sum;
  int4 bo;
  if constexpr (LISTS) {
    int32_t ex[2], tt[2], sm[5];
    const int32_t xs[2] = {c.x | (c.y << 16), c.z | (c.w << 16)};
    const int32_t ys[5] = {part.x, part.y, part.z, part.w, rsw};
    block_scan_sum<WT, 2, 5>(xs, ys, lds, ex, tt, sm);
    bo = boff ? boff[blockIdx.x] : make_int4(sm[0], sm[1], sm[2], sm[3]);
    fs = ex[0];
    dg = ex[1];
    nf = tt[0];
    rs_sum = sm[4];
  } else {
    int32_t ex[1], tt[1], sm[3];
    const int32_t xs[1] = {c.x | (c.y << 16)};
    const int32_t ys[3] = {part.x, part.y, rsw};
    block_scan_sum<WT, 1, 3>(xs, ys, lds, ex, tt, sm);
    bo = boff ? boff[blockIdx.x] : make_int4(sm[0], sm[1], 0, 0);
    fs = ex[0];
    nf = tt[0];
    rs_sum = sm[2];
    if (agg) {
      // no block-sum launch: publish this block's counts (new and old
      // entries, 16 bits each under a flag), then add up those of the blocks
      // before it, waiting for each to appear.  Blocks start in index order,
      // so every block waited on is running or done; the wait is bounded
      // all the same, and a timeout is an error.
      if (t == 0)
        __hip_atomic_store(&agg[blockIdx.x], AGG_FLAG | (uint32_t)tt[0], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      int32_t px = 0, py = 0;
      bool late = false;
      for (int64_t i = t; i < nb_before; i += WT) {
        uint64_t v = __hip_atomic_load(&agg[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int spin = 0; !(v & AGG_FLAG); ++spin) {
          if (spin >= AGG_SPIN_MAX) {
            late = true;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
          v = __hip_atomic_load(&agg[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        px += (int32_t)(v & 0xFFFFu);
        py += (int32_t)((v >> 16) & 0xFFFFu);
      }
      if (late) atomicOr(const_cast<int32_t*>(&st->err), 16);
      for (int off = 32; off > 0; off >>= 1) {
        px += __shfl_xor(px, off, SNK_WAVE);
        py += __shfl_xor(py, off, SNK_WAVE);
      }
      if (lane_id() == 0) {
        red2[t / SNK_WAVE][0] = px;
        red2[t / SNK_WAVE][1] = py;
      }
      __syncthreads();
      bo = make_int4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < WT / SNK_WAVE; ++i) {
        bo.x += red2[i][0];
        bo.y += red2[i][1];
      }
    }
  }
  if (fp_tiled && t == 0) rs_blk[blockIdx.x] = rs_sum;
  // the block's new entries are [bo.x, bo.x + nblk_out); listed in LDS when
  // they fit (block-uniform), so that each thread takes one entry per round
  // and the stores are coalesced
  const int32_t nblk_out = nf & 0xFFFF;
  const bool listed = nblk_out <= EMIT_CAP;
  int64_t qf = bo.x + (fs & 0xFFFF);
  const int64_t qs = bo.y + (fs >> 16);
  int64_t qd = bo.z + (dg & 0xFFFF);
  int64_t qg = bo.w + (dg >> 16);
  uint32_t F = F0;
  if (FP && w < W) {  // the new support and its per-word prefix, for a fused prepare
    // (row-major, or in 16-row tiles when the column emitter reads it)
    const int64_t at = fp_tiled ? fp_tile_index(r0, c0 >> 5, (int64_t)K >> 5) : w;
    FP[at] = make_uint2(F, (uint32_t)qf);
  }

  if (listed) {
    sS[t] = S;
    sq[t] = (int32_t)qs;
    sr[t] = r0;
    sc[t] = c0;
    int32_t o = fs & 0xFFFF;
    for (uint32_t x = F; x; x &= x - 1) ent[o++] = ((uint32_t)t << 5) | (uint32_t)(__ffs(x) - 1);
  } else {
    // a block denser than EMIT_CAP (rare): one thread per word, bit by bit
    for (; F; F &= F - 1) {
      const int b = __ffs(F) - 1;
      if (qf < nnz) {
        const T v = ((S >> b) & 1u) ? vals_ws[qs + __popc(S & ((1u << b) - 1u))] : (T)0;
        int32_t r = r0, cc = c0 + b;
        while (cc >= K) {
          cc -= K;
          ++r;
        }
        row[qf] = r;
        col[qf] = cc;
        vals[qf] = v;
      }
      ++qf;
    }
  }
  if (LISTS && dropped_lin) {
    uint32_t Dw = D;
    while (Dw) {
      const int b = __ffs(Dw) - 1;
      Dw &= Dw - 1;
      if (qd < n_drop) dropped_lin[qd] = pw + b;
      ++qd;
    }
  }
  if (LISTS && grown_lin) {
    uint32_t Gw = G;
    while (Gw) {
      const int b = __ffs(Gw) - 1;
      Gw &= Gw - 1;
      if (qg < n_drop) grown_lin[qg] = pw + b;
      ++qg;
    }
  }
  if (listed) {
    __syncthreads();
    const int32_t lim = (int32_t)std::max<int64_t>(0, std::min<int64_t>(nblk_out, nnz - bo.x));
    // two entries per thread per round, their survivor-value loads in flight
    // together; row and column indices with streaming stores, the values with
    // plain ones (the column emitter of a fused prepare gathers them again)
    for (int32_t j0 = t; j0 < lim; j0 += 2 * WT) {
      int32_t r[2], cc[2];
      bool live[2], surv[2];
      int64_t src[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int32_t j = j0 + u * WT;
        live[u] = j < lim;
        const uint32_t e = ent[live[u] ? j : j0];
        const int wl = (int)(e >> 5), bt = (int)(e & 31u);
        const uint32_t Sw = sS[wl];
        surv[u] = (Sw >> bt) & 1u;
        // a grown entry reads the first element (L1-resident; discarded)
        src[u] = surv[u] ? (int64_t)sq[wl] + __popc(Sw & ((1u << bt) - 1u)) : 0;
        r[u] = sr[wl];
        cc[u] = sc[wl] + bt;
      }
      T v[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) v[u] = vals_ws[src[u]];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (!live[u]) continue;
        while (cc[u] >= K) {
          cc[u] -= K;
          ++r[u];
        }
        const int64_t q = bo.x + j0 + u * WT;
        __builtin_nontemporal_store(r[u], &row[q]);
        __builtin_nontemporal_store(cc[u], &col[q]);
        vals[q] = surv[u] ? v[u] : (T)0;
      }
    }
  }
}

// ====================================================== fused restructure + prepare
// With K and M multiples of 32, rows of F are word-aligned and the plan's
// derived arrays of the new COO come straight from F and its per-word
// prefix counts pw (no sort):
//   rows     row_ptr[s] = pw[s * K/32] (nnz at s = M); the row tiles follow;
//   columns  up to FC_MAX_M rows, k_fp_colemit: one column word of every
//            row staged in LDS, 64-row ballots per column; taller layouts:
//            FT = F transposed in 32 x 32 bit tiles (32 ballots per wave
//            give the 32 column words of two tiles), compacted in
//            column-major order.  Either way the entries come column by
//            column, rows ascending: row_t, col_ptr, and perm = each entry's
//            rank in F, i.e. its row-major index.
struct fuse_ptrs {
  int32_t *row_ptr, *rpart_seg, *rpart_nz, *rcut;
  int32_t *col_ptr, *perm, *row_t, *cpart_seg, *cpart_nz, *ccut;
  int32_t T_row, P_row, T_col, P_col;
};

__device__ __forceinline__ bool bm_failed(const bm_state* st) {
  return st->err != 0 || st->rem_final > 0;
}

constexpr int FP_THREADS = 256;

// Blocks [0, rb): row offsets and row tiles, thread per row s in [0, M]; a
// block with a split row sets res[2] (pinned host memory, cleared by the
// emitter).  Blocks [rb, ..): the bit transpose FT of F and its popcount
// sums per block of WT words of FT (k_fp_temit's blocks), which tsum must
// hold zeroed.  Block j covers column word wc and row words rw0 .. rw0+7
// (two 32 x 32 tiles per wave: 32 ballots give the column words of both),
// so that neighbouring lanes of the block write neighbouring FT words and
// the block's counts fall into a few FT blocks, summed in LDS first.
constexpr int TS_SPAN = 256;  // FT blocks one transpose block can touch, summed in LDS
__global__ __launch_bounds__(FP_THREADS) void k_fp_rows_transpose(
    const bm_state* st, const uint2* __restrict__ FP,
    int32_t M, int32_t K, int64_t nnz, fuse_ptrs f, int32_t rb, int32_t* __restrict__ res,
    uint32_t* __restrict__ FT, int32_t* __restrict__ tsum) {
  __shared__ int32_t tsl[TS_SPAN];
  const int64_t KW = K >> 5, WM = M >> 5;
  if ((int)blockIdx.x < rb) {
    // the FP loads (clamped in range) go out before the state check
    const int64_t s = (int64_t)blockIdx.x * FP_THREADS + threadIdx.x;
    const int32_t fa = (int32_t)FP[(s < M ? s : M - 1) * KW].y;
    const int32_t fb = (int32_t)FP[(s + 1 < M ? s + 1 : M - 1) * KW].y;
    if (bm_failed(st)) return;
    bool any = false;
    if (s < M) {
      const int64_t a = fa;
      const int64_t b = s + 1 < M ? (int64_t)fb : nnz;
      f.row_ptr[s] = (int32_t)a;
      any = tile_cuts(s, a, b, nnz, f.T_row, f.P_row, f.rpart_seg, f.rpart_nz, f.rcut);
    } else if (s == M) {
      f.row_ptr[M] = (int32_t)nnz;
      tile_close(M, nnz, f.P_row, f.rpart_seg, f.rpart_nz, f.rcut);
    }
    const int any_b = __syncthreads_or(any ? 1 : 0);
    if (threadIdx.x == 0 && any_b) store_result(&res[2], 1);
    return;
  }
  const int64_t RWG = cdiv_dev(WM, 8);  // groups of 8 row words per column word
  const int64_t j = (int64_t)blockIdx.x - rb;
  const int64_t wc = j / RWG, rw0 = (j - wc * RWG) * 8;
  const int lane = threadIdx.x & 63, l = lane & 31;
  const int64_t rw = rw0 + 2 * (threadIdx.x >> 6) + (lane >> 5);
  const bool ok = wc < KW && rw < WM;
  const uint32_t w0 = FP[ok ? (rw * 32 + l) * KW + wc : 0].x;  // before the state check
  if (bm_failed(st)) return;
  const uint32_t word = ok ? w0 : 0u;
  uint32_t out = 0;
#pragma unroll
  for (int b = 0; b < 32; ++b) {
    const uint64_t m = __ballot((word >> b) & 1u);  // bit i: row i of the lane's tile
    if (l == b) out = (lane & 32) ? (uint32_t)(m >> 32) : (uint32_t)m;
  }
  const int64_t c = wc * 32 + l;
  if (ok) FT[c * WM + rw] = out;
  // the FT blocks this block's words fall in: [tb_lo, tb_hi] (block-uniform)
  const int64_t rw_last = std::min<int64_t>(rw0 + 7, WM - 1);
  const int64_t tb_lo = (wc * 32 * WM + rw0) / WT;
  const int64_t tb_hi = ((wc * 32 + 31) * WM + rw_last) / WT;
  const bool in_lds = tb_hi - tb_lo < TS_SPAN;
  if (in_lds)
    for (int i = threadIdx.x; i < TS_SPAN; i += FP_THREADS) tsl[i] = 0;
  __syncthreads();
  const int32_t pc = ok ? __popc(out) : 0;
  if (pc) {
    const int64_t tb = (c * WM + rw) / WT;
    if (in_lds) atomicAdd(&tsl[tb - tb_lo], pc);
    else atomicAdd(&tsum[4 * tb], pc);  // .x of the block's int4
  }
  if (in_lds) {
    __syncthreads();
    for (int64_t i = threadIdx.x; i <= tb_hi - tb_lo; i += FP_THREADS)
      if (tsl[i]) atomicAdd(&tsum[4 * (tb_lo + i)], tsl[i]);
  }
}

// Column view: one thread per FT word (column c, rows 32rw ..); rank of its
// first entry = block base + block scan.  Word block tb holds columns
// [tb*WT/WM, ...); workgroup b (dispatched to XCD b mod 8) takes word block
// (b mod 8)*ceil(nbt/8) + b/8, so each XCD gathers the FP lines of one
// contiguous column range.  The gathers of a thread's first TE_FIRST entries
// (the FP word of each entry's row, then its value) go out before the block
// scan, so that their round trips overlap it; further entries (rare) follow
// in batches of EMIT_BATCH.  With cols_here (WM divides WT, so a block holds
// whole columns) the block also writes the column tiles of its columns and
// sets res[3] if one of them is split.
constexpr int TE_FIRST = 4;
template <typename T>
__global__ __launch_bounds__(WT, 8) void k_fp_temit(
    const bm_state* st, const uint32_t* __restrict__ FT, int64_t NT, int64_t nbt, int32_t M,
    int32_t K, const int4* __restrict__ tsum, const int4* __restrict__ toff,
    const uint2* __restrict__ FP, int64_t nnz, fuse_ptrs f, int32_t cols_here,
    int32_t* __restrict__ res, const T* __restrict__ vals, T* __restrict__ vals_t) {
  __shared__ int32_t lds[WT / SNK_WAVE * 2];
  __shared__ int32_t cstart[WT];
  const int64_t per_xcd = cdiv_dev(nbt, NUM_XCD);
  const int64_t tb = (int64_t)(blockIdx.x % NUM_XCD) * per_xcd + blockIdx.x / NUM_XCD;
  if (tb >= nbt) return;  // uniform over the block
  const int t = threadIdx.x;
  // loads that depend on nothing first: the thread's FT word and the block
  // sums before it (up to 2 WT of them here), then the state words
  const int64_t i = tb * WT + t;
  const bool valid = i < NT;
  const uint32_t word0 = FT[valid ? i : NT - 1];
  int32_t p0 = 0, p1 = 0;
  if (!toff && tb > 0) {
    p0 = tsum[t < tb ? t : 0].x;
    p1 = tsum[t + WT < tb ? t + WT : 0].x;
  }
  if (bm_failed(st)) return;  // uniform over the grid
  const int64_t KW = K >> 5, WM = M >> 5;
  const uint32_t word = valid ? word0 : 0u;
  // column and row word of the thread's FT word (32-bit division when the
  // words fit)
  int64_t c, c0;
  if (NT + WT <= INT32_MAX) {
    c = (int64_t)((uint32_t)i / (uint32_t)WM);
    c0 = (int64_t)((uint32_t)(tb * WT) / (uint32_t)WM);  // first column of the block (cols_here)
  } else {
    c = i / WM;
    c0 = tb * WT / WM;
  }
  const int64_t rw = i - c * WM;
  const uint32_t below = (1u << (c & 31)) - 1u;
  // the first entries' gathers, unconditional: an unused slot reads the
  // first element (one line, which every CU keeps in its L1; re-reading the
  // thread's own first address instead measured 35% slower, each such read
  // being one more L2 request) and its result is discarded
  int32_t j[TE_FIRST], pos[TE_FIRST];
  T v[TE_FIRST];
  uint32_t rest = word;
  {
    uint2 fp[TE_FIRST];
#pragma unroll
    for (int u = 0; u < TE_FIRST; ++u) {
      j[u] = rest ? __ffs(rest) - 1 : -1;
      rest &= rest - 1;
    }
#pragma unroll
    for (int u = 0; u < TE_FIRST; ++u)
      fp[u] = FP[j[u] >= 0 ? (rw * 32 + j[u]) * KW + (c >> 5) : 0];
#pragma unroll
    for (int u = 0; u < TE_FIRST; ++u) pos[u] = (int32_t)fp[u].y + __popc(fp[u].x & below);
    // all value loads issued back to back (vals_t or not: the new values
    // always exist), waited for only at the stores after the scan
#pragma unroll
    for (int u = 0; u < TE_FIRST; ++u) v[u] = vals[(j[u] >= 0 && pos[u] < nnz) ? pos[u] : 0];
  }
  // this thread's share of the block base (the entries of earlier blocks),
  // reduced by the block together with the scan of its words' counts
  int32_t part = 0;
  if (!toff) {
    part = (t < tb ? p0 : 0) + (t + WT < tb ? p1 : 0);
    for (int64_t k = t + 2 * WT; k < tb; k += 2 * WT) {  // two loads in flight
      const int64_t k2 = k + WT < tb ? k + WT : k;
      const int32_t x = tsum[k].x, y = tsum[k2].x;
      part += k2 != k ? x + y : x;
    }
  }
  int32_t ex1[1], tt1[1], sm1[1];
  {
    const int32_t xs[1] = {(int32_t)__popc(word)};
    const int32_t ys[1] = {part};
    block_scan_sum<WT, 1, 1>(xs, ys, lds, ex1, tt1, sm1);
  }
  const int64_t base = toff ? (int64_t)toff[tb].x : (int64_t)sm1[0];
  const int32_t tot = tt1[0];
  int64_t q = base + ex1[0];
  if (valid && rw == 0) {
    f.col_ptr[c] = (int32_t)q;
    if (cols_here) cstart[c - c0] = (int32_t)q;
  }
  if (valid && i == NT - 1) {
    f.col_ptr[K] = (int32_t)nnz;
    if (cols_here) tile_close(K, nnz, f.P_col, f.cpart_seg, f.cpart_nz, f.ccut);
  }
#pragma unroll
  for (int u = 0; u < TE_FIRST; ++u) {
    if (j[u] >= 0 && q < nnz) {
      f.row_t[q] = (int32_t)(rw * 32 + j[u]);
      f.perm[q] = pos[u];
      if (vals_t) vals_t[q] = v[u];
    }
    q += j[u] >= 0 ? 1 : 0;
  }
  while (rest) {  // words with more than TE_FIRST entries
    int jb[EMIT_BATCH];
    uint2 fp[EMIT_BATCH];
#pragma unroll
    for (int u = 0; u < EMIT_BATCH; ++u) {
      jb[u] = rest ? __ffs(rest) - 1 : -1;
      rest &= rest - 1;
    }
#pragma unroll
    for (int u = 0; u < EMIT_BATCH; ++u)
      fp[u] = jb[u] >= 0 ? FP[(rw * 32 + jb[u]) * KW + (c >> 5)] : make_uint2(0u, 0u);
    int32_t pb[EMIT_BATCH];
    T vb[EMIT_BATCH];
#pragma unroll
    for (int u = 0; u < EMIT_BATCH; ++u) {
      pb[u] = (int32_t)fp[u].y + __popc(fp[u].x & below);
      if (vals_t) vb[u] = (jb[u] >= 0 && pb[u] < nnz) ? vals[pb[u]] : (T)0;
    }
#pragma unroll
    for (int u = 0; u < EMIT_BATCH; ++u) {
      if (jb[u] < 0) break;
      if (q < nnz) {
        f.row_t[q] = (int32_t)(rw * 32 + jb[u]);
        f.perm[q] = pb[u];
        if (vals_t) vals_t[q] = vb[u];
      }
      ++q;
    }
  }
  if (cols_here) {  // the tiles of the block's columns
    __syncthreads();  // publishes cstart
    const int64_t ncol = WT / WM;
    const int64_t s = c0 + t;
    bool any = false;
    if (t < ncol && s < K) {
      const int64_t a = cstart[t];
      const int64_t b = (t + 1 < ncol && s + 1 < K) ? (int64_t)cstart[t + 1] : base + tot;
      any = tile_cuts(s, a, b, nnz, f.T_col, f.P_col, f.cpart_seg, f.cpart_nz, f.ccut);
    }
    if (__ballot(any) != 0 && lane_id() == 0) store_result(&res[3], 1);
  }
}

// Column view straight from F (up to FC_MAX_M rows): workgroup b owns FC_CPB
// columns [ca, ca + FC_CPB) of column word cw = b / FC_SPLIT and stages that
// word of every row (F and its row-major prefix P, from the 16-row tiles of
// FP) in LDS.  Its entries come out in column-major order from 64-row
// ballots of its columns' bits, so no transposed bitmap is written.  Its
// place in the output needs no other workgroup: the entries in columns
// before ca are, summed over rows, the row-major prefix at (r, ca) minus the
// row's start, i.e. sum_r (P(r, cw) + popc(F(r, cw) below ca)) - sum_r
// start(r), the last sum being the row emitter's per-block terms.  A value
// is gathered from the new row-major values at its row-major rank.  Each
// workgroup also writes row_ptr and the row tiles of rows
// [b * rpb, (b + 1) * rpb) (res[2] on a split row), and its columns' col_ptr
// and tiles (res[3] on a split column).
constexpr int FC_THREADS = 512;
constexpr int FC_SPLIT = 4;                       // workgroups per column word
constexpr int FC_CPB = 32 / FC_SPLIT;             // columns per workgroup
constexpr int FC_MAX_CH = FC_MAX_M / SNK_WAVE;    // 64-row chunks at most
constexpr int FC_IPT = FC_CPB * FC_MAX_CH / FC_THREADS;  // (column, chunk) items per thread at most
constexpr int FC_LOAD = 8;                        // row loads per thread in flight
inline size_t fc_lds_bytes(int32_t M) {
  return 8 * (size_t)FC_CPB * (size_t)cdiv((int64_t)M, SNK_WAVE) + 8 * (size_t)M;
}
template <typename T>
__global__ __launch_bounds__(FC_THREADS) void k_fp_colemit(
    const bm_state* st, const uint2* __restrict__ FP, const int32_t* __restrict__ rs_blk,
    int64_t nb, int32_t M, int32_t K, int64_t nnz, fuse_ptrs f, int32_t rpb,
    int32_t* __restrict__ res, const T* __restrict__ vals, T* __restrict__ vals_t) {
  // dynamic LDS (fc_lds_bytes): the 64-row masks of the columns, then F and
  // P of every row
  extern __shared__ uint64_t fc_smem[];
  __shared__ int32_t lds[FC_THREADS / SNK_WAVE * 3];
  __shared__ int32_t cstart[FC_CPB];
  const int nch = (M + SNK_WAVE - 1) / SNK_WAVE;
  uint64_t* sm = fc_smem;  // [FC_CPB][nch]
  uint32_t* sF = reinterpret_cast<uint32_t*>(fc_smem + FC_CPB * nch);
  int32_t* sP = reinterpret_cast<int32_t*>(sF + M);
  const int t = threadIdx.x, lane = t & (SNK_WAVE - 1), wv = t / SNK_WAVE;
  const int64_t KW = K >> 5;
  const int64_t cw = blockIdx.x / FC_SPLIT;
  const int cb = (int)(blockIdx.x % FC_SPLIT) * FC_CPB;  // first column within the word
  const int64_t ca = cw * 32 + cb;
  const uint32_t lowmask = (1u << cb) - 1u;
  // this workgroup's share of the rows, [row_lo, row_hi]: the start words
  // of its first FC_THREADS go out with the staging loads, and so do the row
  // emitter's terms (two per thread here; indices clamped in range)
  const int64_t row_lo = (int64_t)blockIdx.x * rpb;
  const int64_t row_hi = std::min<int64_t>(row_lo + rpb - 1, M);
  const int64_t s_row = row_lo + t;
  const int64_t sr0 = s_row < M ? s_row : M - 1, sr1 = s_row + 1 < M ? s_row + 1 : M - 1;
  const int32_t ra = (int32_t)FP[fp_tile_index(sr0, 0, KW)].y;
  const int32_t rb_ = (int32_t)FP[fp_tile_index(sr1, 0, KW)].y;
  const int32_t rsa = rs_blk[t < nb ? t : 0];
  const int32_t rsb = rs_blk[t + FC_THREADS < nb ? t + FC_THREADS : 0];
  // stage column word cw of every row (a wave's lanes hold 64 consecutive
  // rows, so the 64-row ballots of the columns' bits are taken on the loaded
  // words); each thread's share of the base.  Tile indices in 32 bits (the
  // whole FP array fits: M * K/32 < 2^31 words).
  int64_t part = 0;
  const uint32_t tile_stride = 16u * (uint32_t)KW, cw16 = 16u * (uint32_t)cw;
  for (int r0 = t; r0 - lane < M; r0 += FC_LOAD * FC_THREADS) {
    uint2 x[FC_LOAD];
#pragma unroll
    for (int u = 0; u < FC_LOAD; ++u) {
      const int r = r0 + u * FC_THREADS;
      const uint32_t rr = (uint32_t)(r < M ? r : M - 1);
      x[u] = FP[(rr >> 4) * tile_stride + cw16 + (rr & 15u)];
    }
#pragma unroll
    for (int u = 0; u < FC_LOAD; ++u) {
      const int r = r0 + u * FC_THREADS;
      const int h = (r - lane) / SNK_WAVE;  // the wave's chunk (uniform)
      if (h >= nch) break;
      const uint32_t fr = r < M ? x[u].x : 0u;
      if (r < M) {
        sF[r] = fr;
        sP[r] = (int32_t)x[u].y;
        part += (int64_t)x[u].y + __popc(fr & lowmask);
      }
      const uint32_t fb = fr >> cb;  // the workgroup's columns in the low bits
      uint64_t mine_m = 0;           // lane j keeps column j's mask
#pragma unroll
      for (int j = 0; j < FC_CPB; ++j) {
        const uint64_t m = __ballot(fb & (1u << j));
        mine_m = lane == j ? m : mine_m;
      }
      if (lane < FC_CPB) sm[lane * nch + h] = mine_m;
    }
  }
  // minus this thread's share of the row starts' sum
  part -= (t < nb ? rsa : 0) + (t + FC_THREADS < nb ? rsb : 0);
  for (int64_t i = t + 2 * FC_THREADS; i < nb; i += FC_THREADS) part -= rs_blk[i];
  if (bm_failed(st)) {  // uniform over the grid; an error raised after the
    // row emitter reported the state (a late block count) is reported here
    if (blockIdx.x == 0 && t == 0) store_result(&res[0], st->err);
    return;
  }
  __syncthreads();
  // (column, chunk) items in column-major order, ipt (<= FC_IPT) consecutive
  // ones per thread: one block scan of their counts, the base reduced with it
  // (as its low 16 bits and the rest: both sums fit 32 bits)
  const int nit = FC_CPB * nch;
  const int ipt = (nit + FC_THREADS - 1) / FC_THREADS;
  const int it0 = t * ipt;
  int32_t mine = 0;
#pragma unroll
  for (int k = 0; k < FC_IPT; ++k) {
    const int it = it0 + k;
    if (k < ipt && it < nit) mine += __popcll(sm[it]);
  }
  int32_t ex1[1], tt1[1], sm1[2];
  {
    const int32_t xs[1] = {mine};
    const int32_t ys[2] = {(int32_t)(part & 0xFFFF), (int32_t)(part >> 16)};
    block_scan_sum<FC_THREADS, 1, 2>(xs, ys, lds, ex1, tt1, sm1);
  }
  const int64_t base = (int64_t)sm1[0] + ((int64_t)sm1[1] << 16);
  const int32_t tot = tt1[0];
  int64_t q = base + ex1[0];
#pragma unroll
  for (int k = 0; k < FC_IPT; ++k) {
    const int it = it0 + k;
    if (k >= ipt || it >= nit) break;
    const int j = it / nch, h = it - j * nch;
    if (h == 0) {  // the column's first entry
      f.col_ptr[ca + j] = (int32_t)q;
      cstart[j] = (int32_t)q;
    }
    const uint32_t below = (1u << (cb + j)) - 1u;
    uint64_t m = sm[it];
    // the item's entries (rows ascending), four value gathers in flight
    while (m) {
      int rr[4];
      int32_t pos[4];
      T v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        rr[u] = m ? h * SNK_WAVE + (__ffsll((long long)m) - 1) : -1;
        m &= m - 1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        pos[u] = rr[u] >= 0 ? sP[rr[u]] + __popc(sF[rr[u]] & below) : 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = vals[pos[u] < nnz ? pos[u] : 0];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (rr[u] < 0) break;
        if (q < nnz) {
          f.row_t[q] = rr[u];
          f.perm[q] = pos[u];
          if (vals_t) vals_t[q] = v[u];
        }
        ++q;
      }
    }
  }
  __syncthreads();  // publishes cstart
  bool any = false;
  if (t < FC_CPB) {
    const int64_t c = ca + t;
    const int64_t a = cstart[t];
    const int64_t b = t + 1 < FC_CPB ? (int64_t)cstart[t + 1] : base + tot;
    any = tile_cuts(c, a, b, nnz, f.T_col, f.P_col, f.cpart_seg, f.cpart_nz, f.ccut);
    if (c == K - 1) {
      f.col_ptr[K] = (int32_t)nnz;
      tile_close(K, nnz, f.P_col, f.cpart_seg, f.cpart_nz, f.ccut);
    }
  }
  if (__ballot(any) != 0 && lane == 0) store_result(&res[3], 1);
  bool any_r = false;
  for (int64_t sr = s_row; sr <= row_hi; sr += FC_THREADS) {
    if (sr < M) {
      const bool first = sr == s_row;  // its start words were loaded up front
      const int32_t a = first ? ra : (int32_t)FP[fp_tile_index(sr, 0, KW)].y;
      const int64_t b = sr + 1 < M ? (int64_t)(first ? rb_ : (int32_t)FP[fp_tile_index(sr + 1, 0, KW)].y)
                                   : nnz;
      f.row_ptr[sr] = a;
      any_r |= tile_cuts(sr, a, b, nnz, f.T_row, f.P_row, f.rpart_seg, f.rpart_nz, f.rcut);
    } else {
      f.row_ptr[M] = (int32_t)nnz;
      tile_close(M, nnz, f.P_row, f.rpart_seg, f.rpart_nz, f.rcut);
    }
  }
  if (__ballot(any_r) != 0 && lane == 0) store_result(&res[2], 1);
}

// Column tiles, thread per column s in [0, K] (shapes whose columns straddle
// the emitter's word blocks); a block with a split column sets res[3].
__global__ __launch_bounds__(FP_THREADS) void k_fp_cols(const bm_state* st, int32_t K,
                                                        int64_t nnz, fuse_ptrs f,
                                                        int32_t* __restrict__ res) {
  if (bm_failed(st)) return;
  const int64_t s = (int64_t)blockIdx.x * FP_THREADS + threadIdx.x;
  bool any = false;
  if (s < K) any = tile_cuts(s, f.col_ptr[s], f.col_ptr[s + 1], nnz, f.T_col, f.P_col,
                             f.cpart_seg, f.cpart_nz, f.ccut);
  else if (s == K) tile_close(K, nnz, f.P_col, f.cpart_seg, f.cpart_nz, f.ccut);
  const int any_b = __syncthreads_or(any ? 1 : 0);
  if (threadIdx.x == 0 && any_b) store_result(&res[3], 1);
}

// ------------------------------------------------------------------ host
struct bm_layout {
  int64_t nblk, W, nb, NT, nbt, rb, cbk;
  size_t res, state, cnt_eq, base_eq, sup, dropb, grown, vals, bsum, boff, rs;
  size_t fp, ft, tsum, toff, total;  // fused prepare
  int64_t nreg, rwg;                  // regions and bucketing workgroups (0: chunk 0 atomic)
  size_t cand, tab;
};

bm_layout make_layout(int32_t M, int32_t K, int64_t nnz) {
  bm_layout L{};
  L.nblk = std::max<int64_t>(1, cdiv(nnz, BE));
  L.W = cdiv((int64_t)M * K, 32);
  L.nb = std::max<int64_t>(1, cdiv(L.W, WT));
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.res = take(4 * RESULT_WORDS);  // result words when no pinned host words are given
  L.state = take(sizeof(bm_state));
  L.cnt_eq = take(4 * (size_t)L.nblk);
  L.base_eq = take(4 * (size_t)L.nblk);
  L.sup = take(4 * (size_t)L.W);
  L.dropb = take(4 * (size_t)L.W);
  L.grown = take(4 * (size_t)L.W);
  L.vals = take(4 * (size_t)std::max<int64_t>(nnz, 1));
  L.bsum = take(16 * (size_t)L.nb);
  L.boff = take(16 * (size_t)L.nb);
  L.rs = take(4 * (size_t)L.nb);
  L.NT = (int64_t)K * cdiv(M, 32);
  L.nbt = std::max<int64_t>(1, cdiv(L.NT, WT));
  L.rb = cdiv((int64_t)M + 1, FP_THREADS);
  L.cbk = cdiv((int64_t)K + 1, FP_THREADS);
  L.fp = take(8 * (size_t)L.W);
  L.ft = take(4 * (size_t)L.NT);
  L.tsum = take(16 * (size_t)L.nbt);
  L.toff = take(16 * (size_t)L.nbt);
  // chunk 0 by region: up to 2^26 positions and n_drop <= nnz (bucketing
  // workgroups capped at RB_MAXWG)
  const int64_t MK = (int64_t)M * K;
  L.nreg = cdiv(MK, (int64_t)1 << RB_SHIFT);
  L.rwg = (MK <= ((int64_t)1 << 26) && L.nreg <= RB_MAXREG)
              ? std::min<int64_t>(cdiv(nnz, RB_CH), RB_MAXWG) : 0;
  L.cand = take(4 * (size_t)L.rwg * RB_CH);
  L.tab = take(4 * (size_t)L.rwg * (size_t)(L.nreg + 1));
  L.total = o;
  return L;
}

// Grid-wide regrow chunks before the finisher: the ones riding on the select
// kernels, plus stand-alone ones while the expected remainder
// n_drop * (1 - q)^c stays above what one workgroup finishes quickly (q: a
// lower bound on the acceptance rate).
double accept_bound(int64_t MK, int64_t nnz, int64_t n_drop) {
  return std::max(0.5, 1.0 - (double)(nnz + n_drop) / (double)MK);
}

int32_t grid_chunks(int64_t MK, int64_t nnz, int64_t n_drop, int32_t riding) {
  const double q = accept_bound(MK, nnz, n_drop);
  int32_t c = riding;
  double rem = (double)n_drop;
  for (int i = 0; i < riding; ++i) rem *= 1.0 - q;
  while (rem > 2048.0 && c < SLOTS) {
    rem *= 1.0 - q;
    ++c;
  }
  return c;
}

// One restructuring step; with `fuse` non-NULL the plan arrays of the new
// COO are built as well and *splits receives the two split flags.
template <typename T>
snack_status run(int32_t* row, int32_t* col, T* vals, int32_t M, int32_t K, int64_t nnz,
                 int64_t n_drop, uint64_t seed, uint64_t step, int64_t* dropped_lin,
                 int64_t* grown_lin, char* ws, result_words& rw, hipStream_t s,
                 const fuse_ptrs* fuse, int32_t* splits, T* vals_t) {
  const bm_layout L = make_layout(M, K, nnz);
  bm_state* st = (bm_state*)(ws + L.state);
  int32_t* cnt_eq = (int32_t*)(ws + L.cnt_eq);
  int32_t* base_eq = (int32_t*)(ws + L.base_eq);
  uint32_t* sup = (uint32_t*)(ws + L.sup);
  uint32_t* dropb = (uint32_t*)(ws + L.dropb);
  uint32_t* grown = (uint32_t*)(ws + L.grown);
  T* vals_ws = (T*)(ws + L.vals);
  int4* bsum = (int4*)(ws + L.bsum);
  int4* boff = (int4*)(ws + L.boff);
  const uint64_t MK = (uint64_t)M * (uint64_t)K;
  const uint64_t stream = sm64_mix(seed + (step + 1) * SM64_GAMMA);
  const int32_t nd = (int32_t)n_drop;
  const dim3 eb((unsigned)L.nblk), et(BT);

  if (!rw.dev) rw.dev = (int32_t*)(ws + L.res);
  int32_t* res_dev = rw.dev;
  if (results_begin(rw, 4, s) != hipSuccess) return SNACK_E_HIP;
  uint2* FP = fuse ? (uint2*)(ws + L.fp) : nullptr;

  // the column emitter when its rows fit in LDS (then no transposed bitmap
  // and no transpose block sums to clear)
  const bool colemit = fuse && M <= FC_MAX_M && (int64_t)M * (K / 32) < ((int64_t)1 << 31);
  // with the column emitter and no lists, the row emitter finds its block
  // bases from the counts earlier blocks publish (no block-sum launch); the
  // published counts, over the block-sum area, start cleared
  const bool agg_path = colemit && !dropped_lin && !grown_lin && L.nb <= PREFIX_INBLOCK_MAX;
  int32_t* tsum_zero = fuse && !colemit ? (int32_t*)(ws + L.tsum)
                       : agg_path      ? (int32_t*)(ws + L.bsum) : nullptr;
  const int64_t nzero = fuse && !colemit ? 4 * L.nbt : agg_path ? 2 * L.nb : 0;
  hipLaunchKernelGGL(k_bi_init, dim3((unsigned)cdiv(std::max<int64_t>(4 * HREPL * 256, nzero), 256)),
                     dim3(256), 0, s, st, tsum_zero, nzero);
  const int32_t vec_ok = ((uintptr_t)row % 16 == 0 && (uintptr_t)col % 16 == 0 &&
                          (uintptr_t)vals % (4 * sizeof(T)) == 0) ? 1 : 0;
  const int passes = sizeof(T) == 2 ? 2 : 4;
  const int top = 8 * (passes - 1);
  // chunk 0 bucketed by region when the layout has room for its n_drop
  const int64_t nwg = cdiv(n_drop, (int64_t)RB_CH);
  const bool bucket = L.rwg > 0 && nwg >= 1 && nwg <= L.rwg;  // (n_drop = 0 never gets here)
  uint32_t* cand = (uint32_t*)(ws + L.cand);
  int32_t* tab = (int32_t*)(ws + L.tab);
  hipLaunchKernelGGL(k_bi_build<T>, dim3((unsigned)(L.nblk + (bucket ? nwg : 0))), et, 0, s, row,
                     col, vals, nnz, M, K, L.W, top, vec_ok, st, sup, bucket ? nullptr : grown,
                     vals_ws, L.nblk, stream, MK, nd, (int32_t)L.nreg, cand, tab);
  // entry workgroups plus the workgroups of regrow chunk c, sized for the
  // positions expected to be missing at its start
  const double q = accept_bound((int64_t)MK, nnz, n_drop);
  auto with_chunk = [&](int32_t c) {
    const double rem = (double)n_drop * std::pow(1.0 - q, (double)c);
    const int64_t rb = std::min<int64_t>(1024, std::max<int64_t>(1, (int64_t)(rem / (4 * BT)) + 1));
    return dim3((unsigned)(L.nblk + rb));
  };
  int32_t c = 0;
  for (int p = 1; p < passes; ++p, ++c) {
    const bool by_region = bucket && c == 0;
    const dim3 g = by_region ? dim3((unsigned)(L.nblk + L.nreg)) : with_chunk(c);
    hipLaunchKernelGGL(k_bi_sel<T>, g, et, 0, s, vals, nnz, L.nblk, p, top - 8 * (p - 1),
                       top - 8 * p, nd, c, stream, MK, st, sup, grown, (int32_t)L.nreg,
                       by_region ? (int32_t)nwg : 0, L.W, cand, tab);
  }
  hipLaunchKernelGGL(k_bi_count<T>, with_chunk(c), et, 0, s, vals, nnz, L.nblk, passes - 1, 0, nd,
                     c, stream, MK, st, cnt_eq, sup, grown);
  ++c;
  const bool own_prefix = L.nblk <= PREFIX_INBLOCK_MAX;
  if (!own_prefix)
    hipLaunchKernelGGL(k_bi_eq_scan, dim3(1), dim3(1024), 0, s, cnt_eq, base_eq, L.nblk);
  // when the drop kernel's chunk is the last grid-wide one, a single
  // workgroup of it also finishes the tail, overlapping the drop work
  const int32_t total = grid_chunks((int64_t)MK, nnz, n_drop, c + 1);
  const bool tail = total == c + 1;
  hipLaunchKernelGGL(k_bi_drop<T>, tail ? dim3((unsigned)(L.nblk + 1)) : with_chunk(c), et, 0, s,
                     row, col, vals, nnz, L.nblk, M, K, L.W, passes - 1, cnt_eq,
                     own_prefix ? nullptr : base_eq, nd, c, stream, MK, st, dropb, sup, grown,
                     tail ? 1 : 0);
  ++c;
  if (!tail) {
    const unsigned cb = (unsigned)std::min<int64_t>(1024, std::max<int64_t>(1, cdiv(n_drop, BT)));
    for (; c < total; ++c)
      hipLaunchKernelGGL(k_bi_chunk, dim3(cb), dim3(BT), 0, s, c, stream, MK, nd, st, sup, grown);
    hipLaunchKernelGGL(k_bi_finish, dim3(1), dim3(FT), 0, s, c, stream, MK, nd, st, sup, grown);
  }
  const bool own_base = L.nb <= PREFIX_INBLOCK_MAX;
  if (!agg_path) {
    hipLaunchKernelGGL(k_bi_wsum, dim3((unsigned)L.nb), dim3(WT), 0, s, sup, dropb, grown, L.W,
                       bsum);
    if (!own_base) hipLaunchKernelGGL(k_bi_bscan, dim3(1), dim3(1024), 0, s, bsum, boff, L.nb);
  }
  // the column emitter (a few columns per workgroup, their column word of
  // every row staged in LDS) when the rows fit; else transpose + emit
  const int32_t fp_tiled = colemit ? 1 : 0;
  int32_t* rs_blk = (int32_t*)(ws + L.rs);
  if (dropped_lin || grown_lin)
    hipLaunchKernelGGL((k_bi_emit<T, true>), dim3((unsigned)L.nb), dim3(WT), 0, s, sup, dropb,
                       grown, L.W, bsum, own_base ? nullptr : boff, vals_ws, K,
                       (int32_t)(MK + 32 <= (1ull << 32)), nnz, n_drop, st, res_dev, FP,
                       fp_tiled, rs_blk, nullptr, row, col, vals, dropped_lin, grown_lin);
  else
    hipLaunchKernelGGL((k_bi_emit<T, false>), dim3((unsigned)L.nb), dim3(WT), 0, s, sup, dropb,
                       grown, L.W, bsum, own_base ? nullptr : boff, vals_ws, K,
                       (int32_t)(MK + 32 <= (1ull << 32)), nnz, n_drop, st, res_dev, FP,
                       fp_tiled, rs_blk, agg_path ? (uint64_t*)(ws + L.bsum) : nullptr, row, col,
                       vals, nullptr, nullptr);
  if (colemit) {
    const int64_t nblk = (int64_t)(K / 32) * FC_SPLIT;
    const int32_t rpb = (int32_t)cdiv((int64_t)M + 1, nblk);
    hipLaunchKernelGGL(k_fp_colemit<T>, dim3((unsigned)nblk), dim3(FC_THREADS),
                       (unsigned)fc_lds_bytes(M), s, st, FP, rs_blk, L.nb, M, K, nnz, *fuse,
                       rpb, res_dev, (const T*)vals, vals_t);
  } else if (fuse) {
    uint32_t* FT = (uint32_t*)(ws + L.ft);
    int4* tsum = (int4*)(ws + L.tsum);
    int4* toff = (int4*)(ws + L.toff);
    const int64_t tblk = (int64_t)(K / 32) * cdiv((int64_t)(M / 32), 8);
    hipLaunchKernelGGL(k_fp_rows_transpose, dim3((unsigned)(L.rb + tblk)), dim3(FP_THREADS), 0,
                       s, st, FP, M, K, nnz, *fuse, (int32_t)L.rb, res_dev, FT, (int32_t*)tsum);
    const bool own_t = L.nbt <= PREFIX_INBLOCK_MAX;
    if (!own_t) hipLaunchKernelGGL(k_bi_bscan, dim3(1), dim3(1024), 0, s, tsum, toff, L.nbt);
    const int32_t cols_here = (WT % (M / 32)) == 0 ? 1 : 0;
    hipLaunchKernelGGL(k_fp_temit<T>, dim3((unsigned)(NUM_XCD * cdiv(L.nbt, NUM_XCD))),
                       dim3(WT), 0, s, st, FT, L.NT, L.nbt, M, K, tsum, own_t ? nullptr : toff,
                       FP, nnz, *fuse, cols_here, res_dev, (const T*)vals, vals_t);
    if (!cols_here)
      hipLaunchKernelGGL(k_fp_cols, dim3((unsigned)L.cbk), dim3(FP_THREADS), 0, s, st, K, nnz,
                         *fuse, res_dev);
  }
  if (hipGetLastError() != hipSuccess || results_wait(rw, 4, s) != hipSuccess)
    return SNACK_E_HIP;
  const int32_t* res_host = rw.words();
  const int32_t err = res_host[0], missing = res_host[1];
  if (err == INT32_MIN) return SNACK_E_HIP;
  if (err & 1) return SNACK_E_NAN;
  if (err & 2) return SNACK_E_COO_RANGE;
  if (err & 4) return SNACK_E_COO_ORDER;
  if (err & 16) return SNACK_E_HIP;  // a block count never appeared (bounded wait)
  if ((err & 8) || missing > 0) return SNACK_E_COUNT;
  if (fuse) {
    if (res_host[2] == INT32_MIN || res_host[3] == INT32_MIN) return SNACK_E_HIP;
    splits[0] = res_host[2];
    splits[1] = res_host[3];
  }
  return SNACK_OK;
}

}  // namespace

// Density <= 1/4 (every chunk then takes at least half of what it draws,
// up to duplicates) and three bitmaps within ~16 bytes per entry + 4 MB.
bool prune_bitmap_ok(int32_t M, int32_t K, int64_t nnz) {
  const int64_t MK = (int64_t)M * K;
  return nnz > 0 && 4 * nnz <= MK && cdiv(MK, 32) <= 4 * nnz + (1 << 20);
}

size_t prune_bitmap_ws_bytes(int32_t M, int32_t K, int64_t nnz) {
  return make_layout(M, K, nnz).total;
}

snack_status prune_bitmap(int32_t* row, int32_t* col, void* vals, snack_dtype dt, int32_t M,
                          int32_t K, int64_t nnz, int64_t n_drop, uint64_t seed, uint64_t step,
                          int64_t* dropped_lin, int64_t* grown_lin, void* ws, hipStream_t s) {
  result_words rw;  // device words in the workspace, read back by a copy
  if (dt == SNACK_F32)
    return run<float>(row, col, (float*)vals, M, K, nnz, n_drop, seed, step, dropped_lin,
                      grown_lin, (char*)ws, rw, s, nullptr, nullptr, nullptr);
  return run<bf16>(row, col, (bf16*)vals, M, K, nnz, n_drop, seed, step, dropped_lin, grown_lin,
                   (char*)ws, rw, s, nullptr, nullptr, nullptr);
}

bool prune_bitmap_fused_ok(int32_t M, int32_t K, int64_t nnz) {
  return prune_bitmap_ok(M, K, nnz) && M % 32 == 0 && K % 32 == 0;
}

snack_status prune_bitmap_prepared(snack_plan* plan, int32_t* row, int32_t* col, void* vals,
                                   void* vals_t, snack_dtype dt, int64_t n_drop, uint64_t seed,
                                   uint64_t step, int64_t* dropped_lin, int64_t* grown_lin,
                                   void* ws, result_words& rw, hipStream_t s) {
  char* a = (char*)plan->arena;
  auto arr = [&](int which) { return (int32_t*)(a + plan->off[which]); };
  fuse_ptrs f{arr(SNACK_ARR_ROW_PTR), arr(SNACK_ARR_RPART_SEG), arr(SNACK_ARR_RPART_NZ),
              arr(SNACK_ARR_RCUT), arr(SNACK_ARR_COL_PTR), arr(SNACK_ARR_PERM),
              arr(SNACK_ARR_ROW_T), arr(SNACK_ARR_CPART_SEG), arr(SNACK_ARR_CPART_NZ),
              arr(SNACK_ARR_CCUT), plan->tile_row, plan->P_row, plan->tile_col, plan->P_col};
  int32_t splits[2] = {0, 0};
  plan->prepared = 0;
  const snack_status st =
      dt == SNACK_F32
          ? run<float>(row, col, (float*)vals, plan->M, plan->K, plan->nnz, n_drop, seed, step,
                       dropped_lin, grown_lin, (char*)ws, rw, s, &f, splits, (float*)vals_t)
          : run<bf16>(row, col, (bf16*)vals, plan->M, plan->K, plan->nnz, n_drop, seed, step,
                      dropped_lin, grown_lin, (char*)ws, rw, s, &f, splits, (bf16*)vals_t);
  if (st != SNACK_OK) return st;
  plan->row = row;
  plan->col = col;
  plan->has_split_row = splits[0];
  plan->has_split_col = splits[1];
  plan->prepared = 1;
  return SNACK_OK;
}

}  // namespace snk
