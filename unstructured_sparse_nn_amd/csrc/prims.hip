// prims.hip -- device-wide exclusive scan and stable LSD radix sort (gfx950).
//
// Both are building blocks of the layer's preprocessing: the column view is a
// stable sort of the entries by column, and the prune/regrow step sorts
// candidate positions and counts accepted ones with scans.  Deterministic:
// integer arithmetic only, no order-dependent atomics.
#include <chrono>
#include <climits>
#include <cstdlib>

#include "common.h"
#include "internal.h"

namespace snk {

// ============================================================== scan
constexpr int SCAN_THREADS = 256;
constexpr int SCAN_PER_THREAD = 4;
constexpr int SCAN_BLOCK = SCAN_THREADS * SCAN_PER_THREAD;  // 1024 items

__device__ __forceinline__ int32_t wave_incl_scan(int32_t x) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < SNK_WAVE; d <<= 1) {
    int32_t y = __shfl_up(x, d, SNK_WAVE);
    if (l >= d) x += y;
  }
  return x;
}

// Exclusive scan of one value per thread over a 256-thread block; returns the
// exclusive prefix and writes the block total to *total.
__device__ __forceinline__ int32_t block_excl_scan(int32_t x, int32_t* lds4, int32_t* total) {
  const int w = threadIdx.x / SNK_WAVE;
  const int l = lane_id();
  int32_t inc = wave_incl_scan(x);
  if (l == SNK_WAVE - 1) lds4[w] = inc;
  __syncthreads();
  int32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < SCAN_THREADS / SNK_WAVE; ++i) {
    int32_t t = lds4[i];
    if (i < w) base += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + inc - x;
}

__global__ __launch_bounds__(SCAN_THREADS) void k_block_reduce(const int32_t* __restrict__ in,
                                                               int64_t n,
                                                               int32_t* __restrict__ sums) {
  __shared__ int32_t lds4[SCAN_THREADS / SNK_WAVE];
  int64_t base = (int64_t)blockIdx.x * SCAN_BLOCK + (int64_t)threadIdx.x * SCAN_PER_THREAD;
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < SCAN_PER_THREAD; ++i)
    if (base + i < n) s += in[base + i];
  int32_t tot;
  block_excl_scan(s, lds4, &tot);
  if (threadIdx.x == 0) sums[blockIdx.x] = tot;
}

// One block scans the per-block sums in place (any count, chunk by chunk).
__global__ __launch_bounds__(SCAN_THREADS) void k_scan_sums(int32_t* __restrict__ sums,
                                                            int64_t nb,
                                                            int32_t* __restrict__ total) {
  __shared__ int32_t lds4[SCAN_THREADS / SNK_WAVE];
  int32_t carry = 0;
  for (int64_t c = 0; c < nb; c += SCAN_THREADS) {
    int64_t i = c + threadIdx.x;
    int32_t x = i < nb ? sums[i] : 0;
    int32_t tot;
    int32_t ex = block_excl_scan(x, lds4, &tot);
    if (i < nb) sums[i] = carry + ex;
    carry += tot;
  }
  if (total && threadIdx.x == 0) *total = carry;
}

__global__ __launch_bounds__(SCAN_THREADS) void k_block_scan(const int32_t* in, int32_t* out,
                                                             int64_t n,
                                                             const int32_t* __restrict__ offs) {
  __shared__ int32_t lds4[SCAN_THREADS / SNK_WAVE];
  int64_t base = (int64_t)blockIdx.x * SCAN_BLOCK + (int64_t)threadIdx.x * SCAN_PER_THREAD;
  int32_t v[SCAN_PER_THREAD];
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < SCAN_PER_THREAD; ++i) {
    v[i] = base + i < n ? in[base + i] : 0;
    s += v[i];
  }
  int32_t tot;
  int32_t ex = block_excl_scan(s, lds4, &tot) + offs[blockIdx.x];
#pragma unroll
  for (int i = 0; i < SCAN_PER_THREAD; ++i) {
    if (base + i < n) out[base + i] = ex;
    ex += v[i];
  }
}

__global__ void k_zero_i32(int32_t* p) { *p = 0; }

// One workgroup scans up to SCAN_SINGLE_MAX elements in coalesced chunks of
// 1024 (one element per thread), carrying the running total between chunks.
// Saves two launches against the three-kernel scan on small arrays.
constexpr int64_t SCAN_SINGLE_MAX = 1 << 15;
constexpr int SCAN_SINGLE_THREADS = 1024;

__global__ __launch_bounds__(SCAN_SINGLE_THREADS) void k_scan_single(const int32_t* in,
                                                                     int32_t* out, int64_t n,
                                                                     int32_t* __restrict__ total) {
  __shared__ int32_t lds[SCAN_SINGLE_THREADS / SNK_WAVE];
  int32_t carry = 0;
  for (int64_t c = 0; c < n; c += SCAN_SINGLE_THREADS) {
    const int64_t i = c + threadIdx.x;
    const int32_t v = i < n ? in[i] : 0;
    int32_t tot;
    const int32_t ex = block_excl_scan_i32<SCAN_SINGLE_THREADS>(v, lds, &tot);
    if (i < n) out[i] = carry + ex;
    carry += tot;
  }
  if (total && threadIdx.x == 0) *total = carry;
}

size_t scan_tmp_bytes(int64_t n) {
  return align_up(sizeof(int32_t) * (size_t)std::max<int64_t>(1, cdiv(n, SCAN_BLOCK)), 256);
}

hipError_t exclusive_scan_i32(const int32_t* in, int32_t* out, int64_t n, int32_t* total,
                              void* tmp, hipStream_t s) {
  if (n <= 0) {
    if (total) hipLaunchKernelGGL(k_zero_i32, dim3(1), dim3(1), 0, s, total);
    return hipGetLastError();
  }
  if (n <= SCAN_SINGLE_MAX) {
    hipLaunchKernelGGL(k_scan_single, dim3(1), dim3(SCAN_SINGLE_THREADS), 0, s, in, out, n,
                       total);
    return hipGetLastError();
  }
  int64_t nb = cdiv(n, SCAN_BLOCK);
  int32_t* sums = (int32_t*)tmp;
  hipLaunchKernelGGL(k_block_reduce, dim3((unsigned)nb), dim3(SCAN_THREADS), 0, s, in, n, sums);
  hipLaunchKernelGGL(k_scan_sums, dim3(1), dim3(SCAN_THREADS), 0, s, sums, nb, total);
  hipLaunchKernelGGL(k_block_scan, dim3((unsigned)nb), dim3(SCAN_THREADS), 0, s, in, out, n,
                     sums);
  return hipGetLastError();
}

// ============================================================== radix sort
// LSD radix sort, ceil(bits/8) passes of equal digit width (<= 8 bits: a
// 12-bit key takes two 6-bit passes).  Per pass: block histograms, a scan of
// each digit's row over the blocks, and a stable scatter.
constexpr int RS_THREADS = 256;
constexpr int RS_ROUNDS = 8;
constexpr int RS_BLOCK = RS_THREADS * RS_ROUNDS;  // 2048 items per block
constexpr int RS_WAVES = RS_THREADS / SNK_WAVE;

// Lanes of the wave holding the same digit (dbits ballots), restricted to
// lanes with `valid` set.
__device__ __forceinline__ uint64_t digit_peers(uint32_t d, bool valid, int dbits) {
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    if (b < dbits) {
      const uint64_t m = __ballot((d >> b) & 1u);
      peers &= ((d >> b) & 1u) ? m : ~m;
    }
  }
  return peers;
}

// Per-block digit histogram, stored digit-major: hist[d * nblk + blk], so that
// an exclusive scan of hist gives each (digit, block) its stable base offset.
template <typename KT>
__global__ __launch_bounds__(RS_THREADS) void k_radix_hist(const KT* __restrict__ keys, int64_t n,
                                                           int shift, int dbits,
                                                           int32_t* __restrict__ hist,
                                                           int64_t nblk) {
  __shared__ int32_t h[256];
  const int nbins = 1 << dbits;
  const uint32_t dmask = (uint32_t)nbins - 1u;
  h[threadIdx.x] = 0;
  __syncthreads();
  int64_t base = (int64_t)blockIdx.x * RS_BLOCK;
  KT key[RS_ROUNDS];
#pragma unroll
  for (int r = 0; r < RS_ROUNDS; ++r) {
    int64_t i = base + r * RS_THREADS + threadIdx.x;
    key[r] = i < n ? keys[i] : (KT)0;
  }
#pragma unroll
  for (int r = 0; r < RS_ROUNDS; ++r) {
    const int64_t i = base + r * RS_THREADS + threadIdx.x;
    const uint32_t d = (uint32_t)(key[r] >> shift) & dmask;
    const uint64_t peers = digit_peers(d, i < n, dbits);
    if (i < n && __popcll(peers & lanemask_lt()) == 0) atomicAdd(&h[d], __popcll(peers));
  }
  __syncthreads();
  if ((int)threadIdx.x < nbins) hist[(int64_t)threadIdx.x * nblk + blockIdx.x] = h[threadIdx.x];
}

// hist is digit-major [nbins][nblk].  Workgroup d turns row d into exclusive
// prefixes over the blocks (in place) and writes the row total to
// dtotal[d]; the scatter adds the digit's base (sum of smaller digits).
__global__ __launch_bounds__(RS_THREADS) void k_radix_scan_digits(int32_t* __restrict__ hist,
                                                                  int64_t nblk,
                                                                  int32_t* __restrict__ dtotal) {
  __shared__ int32_t lds[RS_THREADS / SNK_WAVE];
  int32_t* row = hist + (int64_t)blockIdx.x * nblk;
  int32_t carry = 0;
  for (int64_t c = 0; c < nblk; c += RS_THREADS) {
    const int64_t i = c + threadIdx.x;
    const int32_t v = i < nblk ? row[i] : 0;
    int32_t tot;
    const int32_t ex = block_excl_scan_i32<RS_THREADS>(v, lds, &tot);
    if (i < nblk) row[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) dtotal[blockIdx.x] = carry;
}

// Stable scatter.  All items of a block are loaded up front (one round
// trip) and ranked in LDS: within a wave, lanes holding the same digit are
// found with ballots and ranked by lane order; per (round, wave, digit)
// counts are turned into block-local offsets by one walk per digit in index
// order.  The block's items are then placed in LDS in digit order and
// written out in coalesced runs.  vin == NULL means value = index.  If
// gsrc != NULL the pass also writes gout[pos] = gsrc[value] (a gather fused
// into the scatter).
template <typename KT>
__global__ __launch_bounds__(RS_THREADS) void k_radix_scatter(
    const KT* __restrict__ kin, const int32_t* __restrict__ vin, KT* __restrict__ kout,
    int32_t* __restrict__ vout, int64_t n, int shift, int dbits, const int32_t* __restrict__ offs,
    int64_t nblk, const int32_t* __restrict__ dtotal, const int32_t* __restrict__ gsrc,
    int32_t* __restrict__ gout) {
  __shared__ int32_t cnt[RS_ROUNDS][RS_WAVES][256];
  __shared__ int32_t dstart[256];  // block-local start of each digit
  __shared__ int32_t gbase[256];   // global position of the block's first item of each digit
  __shared__ KT skey[RS_BLOCK];
  __shared__ int32_t sval[RS_BLOCK];
  __shared__ int32_t sgv[RS_BLOCK];
  __shared__ int32_t lds[RS_WAVES];
  const int t = threadIdx.x;
  const int w = t / SNK_WAVE;
  const int nbins = 1 << dbits;
  const uint32_t dmask = (uint32_t)nbins - 1u;
  const int64_t base = (int64_t)blockIdx.x * RS_BLOCK;
  const int nvalid = (int)std::min<int64_t>(RS_BLOCK, n - base);
  KT key[RS_ROUNDS];
  int32_t val[RS_ROUNDS], gv[RS_ROUNDS];
#pragma unroll
  for (int r = 0; r < RS_ROUNDS; ++r) {
    const int64_t i = base + r * RS_THREADS + t;
    key[r] = i < n ? kin[i] : (KT)0;
    val[r] = i < n ? (vin ? vin[i] : (int32_t)i) : 0;
  }
  if (gsrc) {
#pragma unroll
    for (int r = 0; r < RS_ROUNDS; ++r) gv[r] = base + r * RS_THREADS + t < n ? gsrc[val[r]] : 0;
  }
  const int32_t dt = t < nbins ? dtotal[t] : 0;
  const int32_t off = t < nbins ? offs[(int64_t)t * nblk + blockIdx.x] : 0;
#pragma unroll
  for (int r = 0; r < RS_ROUNDS; ++r)
#pragma unroll
    for (int j = 0; j < RS_WAVES; ++j) cnt[r][j][t] = 0;
  __syncthreads();
  // intra-wave ranks and per (round, wave, digit) counts
  const uint64_t lt = lanemask_lt();
  int32_t rank[RS_ROUNDS];
  uint32_t dig[RS_ROUNDS];
#pragma unroll
  for (int r = 0; r < RS_ROUNDS; ++r) {
    const bool valid = base + r * RS_THREADS + t < n;
    dig[r] = (uint32_t)(key[r] >> shift) & dmask;
    const uint64_t peers = digit_peers(dig[r], valid, dbits);
    rank[r] = __popcll(peers & lt);
    if (valid && rank[r] == 0) cnt[r][w][dig[r]] = __popcll(peers);
  }
  __syncthreads();
  // per digit: exclusive offsets over (round, wave) in index order
  int32_t tot_d = 0;
  if (t < nbins) {
#pragma unroll
    for (int r = 0; r < RS_ROUNDS; ++r)
#pragma unroll
      for (int j = 0; j < RS_WAVES; ++j) {
        const int32_t c = cnt[r][j][t];
        cnt[r][j][t] = tot_d;
        tot_d += c;
      }
  }
  int32_t sum;
  const int32_t ds = block_excl_scan_i32<RS_THREADS>(tot_d, lds, &sum);
  const int32_t db = block_excl_scan_i32<RS_THREADS>(dt, lds, &sum);
  if (t < nbins) {
    dstart[t] = ds;
    gbase[t] = db + off;
  }
  __syncthreads();
  // place the block's items in digit order
#pragma unroll
  for (int r = 0; r < RS_ROUNDS; ++r) {
    if (base + r * RS_THREADS + t < n) {
      const int lp = dstart[dig[r]] + cnt[r][w][dig[r]] + rank[r];
      skey[lp] = key[r];
      sval[lp] = val[r];
      if (gsrc) sgv[lp] = gv[r];
    }
  }
  __syncthreads();
  // coalesced runs out
  for (int slot = t; slot < nvalid; slot += RS_THREADS) {
    const KT k = skey[slot];
    const uint32_t d = (uint32_t)(k >> shift) & dmask;
    const int64_t pos = (int64_t)gbase[d] + (slot - dstart[d]);
    kout[pos] = k;
    vout[pos] = sval[slot];
    if (gsrc) gout[pos] = sgv[slot];
  }
}

size_t radix_tmp_bytes(int64_t n) {
  int64_t nblk = std::max<int64_t>(1, cdiv(n, RS_BLOCK));
  return align_up(sizeof(int32_t) * 256 * (size_t)nblk, 256) + 256 * sizeof(int32_t);
}

// Passes read (keys_in, vals_in) first, then ping-pong between the two
// buffer pairs so that the last pass writes kbuf[0] / vbuf[0].
template <typename KT>
static hipError_t radix_sort(const KT* keys_in, const int32_t* vals_in, KT* const kbuf[2],
                             int32_t* const vbuf[2], int64_t n, int bits, const int32_t* gsrc,
                             int32_t* gout, void* tmp, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int passes = std::max(1, (bits + 7) / 8);
  const int dbits = std::max(1, (bits + passes - 1) / passes);
  const int64_t nblk = cdiv(n, RS_BLOCK);
  int32_t* hist = (int32_t*)tmp;
  int32_t* dtotal = (int32_t*)((char*)tmp + align_up(sizeof(int32_t) * 256 * (size_t)nblk, 256));
  const KT* kin = keys_in;
  const int32_t* vin = vals_in;
  for (int p = 0; p < passes; ++p) {
    const int shift = dbits * p;
    const int o = (passes - 1 - p) & 1;
    const bool last = p == passes - 1;
    hipLaunchKernelGGL(k_radix_hist<KT>, dim3((unsigned)nblk), dim3(RS_THREADS), 0, s, kin, n,
                       shift, dbits, hist, nblk);
    hipLaunchKernelGGL(k_radix_scan_digits, dim3(1u << dbits), dim3(RS_THREADS), 0, s, hist, nblk,
                       dtotal);
    hipLaunchKernelGGL(k_radix_scatter<KT>, dim3((unsigned)nblk), dim3(RS_THREADS), 0, s, kin,
                       vin, kbuf[o], vbuf[o], n, shift, dbits, hist, nblk, dtotal,
                       last ? gsrc : nullptr, last ? gout : nullptr);
    kin = kbuf[o];
    vin = vbuf[o];
  }
  return hipGetLastError();
}

hipError_t radix_sort_u32(const uint32_t* keys_in, const int32_t* vals_in, uint32_t* const kbuf[2],
                          int32_t* const vbuf[2], int64_t n, int bits, const int32_t* gsrc,
                          int32_t* gout, void* tmp, hipStream_t s) {
  return radix_sort<uint32_t>(keys_in, vals_in, kbuf, vbuf, n, bits, gsrc, gout, tmp, s);
}

hipError_t radix_sort_u64(const uint64_t* keys_in, const int32_t* vals_in, uint64_t* const kbuf[2],
                          int32_t* const vbuf[2], int64_t n, int bits, void* tmp, hipStream_t s) {
  return radix_sort<uint64_t>(keys_in, vals_in, kbuf, vbuf, n, bits, nullptr, nullptr, tmp, s);
}

// ============================================================== host results
__global__ void k_fill_words(int32_t* __restrict__ w, int32_t n, int32_t v) {
  if ((int32_t)threadIdx.x < n) w[threadIdx.x] = v;
}

// Completion word of a call: one thread stores the call's token into the
// pinned result words after every earlier kernel of the stream has finished
// (stream order); the host spins on it instead of a blocking stream sync.
__global__ void k_signal(int32_t* __restrict__ flag, int32_t token) {
  __threadfence_system();
  *(volatile int32_t*)flag = token;
}

hipError_t results_begin(result_words& r, int n, hipStream_t s) {
  if (r.host) {
    for (int i = 0; i < n; ++i) r.host[i] = INT32_MIN;
    return hipSuccess;
  }
  for (int i = 0; i < n; ++i) r.local[i] = INT32_MIN;
  hipLaunchKernelGGL(k_fill_words, dim3(1), dim3(64), 0, s, r.dev, (int32_t)n, INT32_MIN);
  return hipGetLastError();
}

hipError_t results_wait(result_words& r, int n, hipStream_t s) {
  if (!r.host) {
    if (hipMemcpyAsync(r.local, r.dev, sizeof(int32_t) * (size_t)n, hipMemcpyDeviceToHost, s) !=
        hipSuccess)
      return hipErrorUnknown;
    return hipStreamSynchronize(s);
  }
  // the token follows the one the previous call left in these words (that
  // call has finished: every call waits for its own token), so no state is
  // kept between calls
  volatile int32_t* flag = r.host + RESULT_DONE_SLOT;
  int32_t token = *flag + 1;
  if (token <= 0) token = 1;
  hipLaunchKernelGGL(k_signal, dim3(1), dim3(1), 0, s, r.dev + RESULT_DONE_SLOT, token);
  if (hipGetLastError() != hipSuccess) return hipStreamSynchronize(s);
  // spin for up to 20 ms (a restructure takes ~0.1 ms), then block: a fault
  // or a slow call still ends in the stream sync and its error
  const auto t0 = std::chrono::steady_clock::now();
  while (*flag != token) {
    if (std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(20))
      return hipStreamSynchronize(s);
    __builtin_ia32_pause();
  }
  return hipSuccess;
}

int32_t* host_words_device(int32_t* host) {
  if (!host) return nullptr;
  void* p = nullptr;
  if (hipHostGetDevicePointer(&p, host, 0) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of a failed lookup
    return nullptr;
  }
  return (int32_t*)p;
}

}  // namespace snk
