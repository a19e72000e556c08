// prune.hip -- one prune-and-regrow step on a device COO weight (gfx950).
//
// The SNACK abstract exposes an API for restructuring connections in dynamic
// sparse training but gives no rule; this library's rule:
//   drop   the n_drop entries smallest in (|value| bits, row*K+col),
//   grow   the first n_drop positions of a SplitMix64 stream (Steele, Lea &
//          Flood, OOPSLA 2014) that are outside the pre-step support and not
//          already taken, value 0,
//   write  survivors + grown back in place, sorted row-major.
// Everything is integer and order-independent, so the mask is bit-exact.
//
// Two device plans share the selection step and give identical results.
//
//   select    radix select of the n_drop-th smallest magnitude, per 8-bit
//             digit (2 passes for bf16, 4 for fp32): blocks build local
//             histograms and add them into replicated global ones, then one
//             workgroup sums them and picks the digit (a block scan);
//   classify  per 1024-entry block: count entries below / at the threshold;
//             one workgroup turns the counts into block offsets, so ties at
//             the threshold are dropped in index order.
//
// Bitmap plan (density <= 1/4 and a support bitmap of modest size):
//   support, dropped and grown positions are bitmaps over the M*K grid;
//   regrow    stream indices are consumed in chunks whose size is the number
//             of positions still missing.  A chunk can then never take more
//             than are missing, so taking every new distinct position of the
//             chunk (test-and-set on the grown bitmap: order-free) yields
//             exactly the first n_drop acceptances of the stream; each chunk
//             shrinks the remainder by the acceptance rate (>= 1/2);
//   write     one pass over the words of (support & ~dropped) | grown writes
//             the new COO in row-major order; a survivor's value comes from
//             its rank in the old support (prefix popcounts).
// Sort plan (anything else):
//   regrow    candidates are drawn C stream positions at a time and radix
//             sorted by position (stable: equal positions keep stream
//             order); a candidate is acceptable if it is the first
//             occurrence of its position and lies outside the old support
//             and the positions taken by earlier chunks (binary searches);
//             the first `need` acceptable ones in stream order are kept (a
//             scan over stream order) and compacted in position order (a
//             scan over sorted order);
//   merge     survivors and grown positions, both sorted, are merged by rank
//             straight into row/col/vals.
// In both plans the kernels that write row/col/vals are launched before the
// single readback and do nothing unless the step is complete and no error
// (NaN, invalid COO) was seen, so the COO is untouched on error.
#include <cstdlib>

#include "common.h"
#include "internal.h"

namespace snk {

constexpr int PR_THREADS = 256;
constexpr int PR_PER_THREAD = 4;
constexpr int PR_BLOCK = PR_THREADS * PR_PER_THREAD;  // entries per classify block
constexpr int PR_REPL = 64;
constexpr int BM_SLOTS = 64;  // chunk records in the ring (a power of two)
constexpr int BM_ACC_REPL = 16;

struct pr_state {
  uint32_t prefix;   // radix-select: magnitude bits fixed so far
  uint32_t mask;
  int32_t need;      // drops still to place among entries matching prefix
  int32_t err;       // 1 = NaN seen
  int32_t got;       // grown positions accepted by committed chunks
  int32_t n_new;     // positions accepted by the latest chunk
  int32_t total_ok;  // acceptable candidates in the latest chunk
  int32_t pad;
  // bitmap plan: ring of regrow-chunk records (stream start, positions still
  // missing at the chunk's start, positions it took)
  int64_t ch_start[64];
  int32_t ch_rem[64];
  int32_t ch_acc[64][16];  // per slot, spread over 16 counters (summed by readers)
  // select histograms, spread over PR_REPL replicas (block b adds into
  // replica b % PR_REPL) so that skewed digits do not serialise on a few
  // global atomics
  int32_t hist[4][PR_REPL][256];
};

// SplitMix64: state advances by the golden gamma; output = variant-13 mix.
__host__ __device__ __forceinline__ uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
constexpr uint64_t SM64_GAMMA = 0x9E3779B97F4A7C15ull;

static inline dim3 g1(int64_t n) {
  return dim3((unsigned)std::max<int64_t>(1, cdiv(n, PR_THREADS)));
}

__device__ __forceinline__ int64_t cdiv_dev(int64_t a, int64_t b) { return (a + b - 1) / b; }

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

// grid: PR_REPL blocks of 256 threads
__global__ void k_pr_init(pr_state* st, int32_t n_drop) {
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < 4; ++p) st->hist[p][blockIdx.x][t] = 0;
  if (blockIdx.x != 0) return;
  for (int i = t; i < BM_SLOTS * BM_ACC_REPL; i += 256) (&st->ch_acc[0][0])[i] = 0;
  if (t == 0) {
    st->prefix = 0;
    st->mask = 0;
    st->need = n_drop;
    st->err = 0;
    st->got = 0;
    st->n_new = 0;
    st->total_ok = 0;
  }
}

// One radix-select pass over the digit at `shift`: each block histograms
// PR_BLOCK magnitudes (wave-aggregated LDS atomics) and adds its histogram
// into replica blockIdx % PR_REPL.  No fence or last-block handshake: the
// digit is picked by k_sel_pick after the kernel boundary (an agent-scope
// fence per block would write back the L2).
template <typename T>
__global__ __launch_bounds__(PR_THREADS) void k_sel_hist(const T* __restrict__ vals, int64_t nnz,
                                                         int shift, int pass, pr_state* st) {
  __shared__ int32_t h[256];
  const int t = threadIdx.x;
  h[t] = 0;
  __syncthreads();
  const uint32_t prefix = st->prefix, mask = st->mask;
  bool nan = false;
  const int64_t base = (int64_t)blockIdx.x * PR_BLOCK;
  uint32_t a[PR_PER_THREAD];
#pragma unroll
  for (int j = 0; j < PR_PER_THREAD; ++j) {
    const int64_t k = base + j * PR_THREADS + t;
    a[j] = k < nnz ? magnitude<T>(raw_bits(vals[k])) : 0u;
  }
#pragma unroll
  for (int j = 0; j < PR_PER_THREAD; ++j) {
    const bool ok = base + j * PR_THREADS + t < nnz;
    nan |= ok && is_nan_mag<T>(a[j]);
    wave_hist_add(h, (a[j] >> shift) & 255u, ok && (a[j] & mask) == prefix);
  }
  if (pass == 0 && nan) atomicOr(&st->err, 1);
  __syncthreads();
  if (h[t]) atomicAdd(&st->hist[pass][blockIdx.x % PR_REPL][t], h[t]);
}

// One workgroup: total histogram of the pass, then the digit holding the
// need-th smallest remaining magnitude (the digit whose inclusive prefix
// count first reaches need).
__global__ __launch_bounds__(256) void k_sel_pick(pr_state* st, int shift, int pass) {
  __shared__ int32_t lds[256 / SNK_WAVE];
  __shared__ int32_t pick[2];
  const int t = threadIdx.x;
  int32_t part[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) part[r] = 0;
#pragma unroll
  for (int r = 0; r < PR_REPL; ++r) part[r & 15] += st->hist[pass][r][t];
  int32_t h = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) h += part[r];
  const int32_t need = st->need;
  int32_t tot;
  const int32_t ex = block_excl_scan_i32<256>(h, lds, &tot);
  if (t == 255) {  // guard: the last digit
    pick[0] = 255;
    pick[1] = ex;
  }
  __syncthreads();
  // exactly one digit has ex < need <= ex + h unless need exceeds the total
  // (not reachable: need <= entries matching the prefix); 255 is the guard
  if (ex < need && need <= ex + h) {
    pick[0] = t;
    pick[1] = ex;
  }
  __syncthreads();
  if (t == 0) {
    st->need = need - pick[1];
    st->prefix |= (uint32_t)pick[0] << shift;
    st->mask |= 255u << shift;
  }
}

// Per block: entries strictly below the threshold magnitude, and at it.
template <typename T>
__global__ __launch_bounds__(PR_THREADS) void k_pr_count(const T* __restrict__ vals, int64_t nnz,
                                                         const pr_state* st,
                                                         int32_t* __restrict__ cnt_lt,
                                                         int32_t* __restrict__ cnt_eq) {
  __shared__ int32_t lds[PR_THREADS / SNK_WAVE];
  const uint32_t tau = st->prefix;
  const int64_t base = (int64_t)blockIdx.x * PR_BLOCK + (int64_t)threadIdx.x * PR_PER_THREAD;
  int32_t lt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < PR_PER_THREAD; ++j) {
    if (base + j < nnz) {
      const uint32_t a = magnitude<T>(raw_bits(vals[base + j]));
      lt += a < tau;
      eq += a == tau;
    }
  }
  int32_t tl, te;
  block_excl_scan_i32<PR_THREADS>(lt, lds, &tl);
  block_excl_scan_i32<PR_THREADS>(eq, lds, &te);
  if (threadIdx.x == 0) {
    cnt_lt[blockIdx.x] = tl;
    cnt_eq[blockIdx.x] = te;
  }
}

// One workgroup: E_b = entries at the threshold in blocks before b; block b
// drops its `lt` entries plus its tied entries of global tie rank < need;
// D_b = drops in blocks before b.
constexpr int PR_DECIDE_THREADS = 1024;
__global__ __launch_bounds__(PR_DECIDE_THREADS) void k_pr_decide(
    const int32_t* __restrict__ cnt_lt, const int32_t* __restrict__ cnt_eq, int64_t nblk,
    const pr_state* st, int32_t* __restrict__ base_eq, int32_t* __restrict__ base_drop) {
  __shared__ int32_t lds[PR_DECIDE_THREADS / SNK_WAVE];
  const int32_t need = st->need;
  int32_t run_eq = 0, run_drop = 0;
  for (int64_t c = 0; c < nblk; c += PR_DECIDE_THREADS) {
    const int64_t b = c + threadIdx.x;
    const int32_t e = b < nblk ? cnt_eq[b] : 0;
    int32_t te;
    const int32_t E = run_eq + block_excl_scan_i32<PR_DECIDE_THREADS>(e, lds, &te);
    const int32_t d = b < nblk ? cnt_lt[b] + min(max(need - E, 0), e) : 0;
    int32_t td;
    const int32_t D = run_drop + block_excl_scan_i32<PR_DECIDE_THREADS>(d, lds, &td);
    if (b < nblk) {
      base_eq[b] = E;
      base_drop[b] = D;
    }
    run_eq += te;
    run_drop += td;
  }
}

// Survivors (in order) with their raw value bits, the dropped list, and the
// sorted pre-step support as linear indices.
template <typename T>
__global__ __launch_bounds__(PR_THREADS) void k_pr_apply(
    const int32_t* __restrict__ row, const int32_t* __restrict__ col, const T* __restrict__ vals,
    int64_t nnz, int32_t K, const pr_state* st, const int32_t* __restrict__ base_eq,
    const int32_t* __restrict__ base_drop, int64_t* __restrict__ sup_lin,
    int64_t* __restrict__ surv_lin, uint32_t* __restrict__ surv_val,
    int64_t* __restrict__ dropped_lin) {
  __shared__ int32_t lds[PR_THREADS / SNK_WAVE];
  const uint32_t tau = st->prefix;
  const int32_t need = st->need;
  const int64_t base = (int64_t)blockIdx.x * PR_BLOCK + (int64_t)threadIdx.x * PR_PER_THREAD;
  uint32_t bits[PR_PER_THREAD], mag[PR_PER_THREAD];
  int32_t eq = 0;
#pragma unroll
  for (int j = 0; j < PR_PER_THREAD; ++j) {
    bits[j] = base + j < nnz ? raw_bits(vals[base + j]) : 0u;
    mag[j] = magnitude<T>(bits[j]);
    eq += (base + j < nnz && mag[j] == tau);
  }
  int32_t tmp;
  int32_t er = base_eq[blockIdx.x] + block_excl_scan_i32<PR_THREADS>(eq, lds, &tmp);
  bool drop[PR_PER_THREAD];
  int32_t nd = 0;
#pragma unroll
  for (int j = 0; j < PR_PER_THREAD; ++j) {
    const bool ok = base + j < nnz;
    const bool is_eq = ok && mag[j] == tau;
    drop[j] = ok && (mag[j] < tau || (is_eq && er < need));
    er += is_eq;
    nd += drop[j];
  }
  int32_t dr = base_drop[blockIdx.x] + block_excl_scan_i32<PR_THREADS>(nd, lds, &tmp);
#pragma unroll
  for (int j = 0; j < PR_PER_THREAD; ++j) {
    const int64_t k = base + j;
    if (k >= nnz) break;
    const int64_t lin = (int64_t)row[k] * K + col[k];
    sup_lin[k] = lin;
    if (drop[j]) {
      if (dropped_lin) dropped_lin[dr] = lin;
      ++dr;
    } else {
      const int64_t pos = k - dr;
      surv_lin[pos] = lin;
      surv_val[pos] = bits[j];
    }
  }
}

// Candidate positions for stream indices base .. base+C-1; thread 0 first
// commits the previous chunk's acceptances.
__global__ __launch_bounds__(PR_THREADS) void k_cand_gen(uint64_t* __restrict__ key, int64_t C,
                                                         uint64_t s, uint64_t base, uint64_t MK,
                                                         pr_state* st) {
  const int64_t t = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
  if (t == 0) {
    st->got += st->n_new;
    st->n_new = 0;
  }
  if (t >= C) return;
  const uint64_t i = base + (uint64_t)t;
  key[t] = __umul64hi(sm64_mix(s + (i + 1) * SM64_GAMMA), MK);
}

__device__ __forceinline__ int64_t lower_bound_i64(const int64_t* __restrict__ a, int64_t n,
                                                   int64_t x) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ bool in_sorted(const int64_t* __restrict__ a, int64_t n, int64_t x) {
  const int64_t i = lower_bound_i64(a, n, x);
  return i < n && a[i] == x;
}

// ok_stream[stream index] = candidate acceptable.
__global__ __launch_bounds__(PR_THREADS) void k_cand_ok(
    const uint64_t* __restrict__ key, const int32_t* __restrict__ val, int64_t C,
    const int64_t* __restrict__ sup, int64_t nnz, const int64_t* __restrict__ acc,
    const pr_state* st, int32_t* __restrict__ ok_stream) {
  const int64_t t = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
  if (t >= C) return;
  const int64_t p = (int64_t)key[t];
  const bool first = t == 0 || key[t - 1] != key[t];
  const bool ok = first && !in_sorted(sup, nnz, p) && !in_sorted(acc, st->got, p);
  ok_stream[val[t]] = ok ? 1 : 0;
}

// sel[t] (sorted order) = acceptable and among the first `need` in stream order.
__global__ __launch_bounds__(PR_THREADS) void k_cand_sel(const int32_t* __restrict__ val,
                                                         int64_t C,
                                                         const int32_t* __restrict__ ok_stream,
                                                         const int32_t* __restrict__ ok_rank,
                                                         const pr_state* st, int32_t n_drop,
                                                         int32_t* __restrict__ sel) {
  const int64_t t = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
  if (t >= C) return;
  const int32_t v = val[t];
  sel[t] = (ok_stream[v] && ok_rank[v] < n_drop - st->got) ? 1 : 0;
}

// Selected positions in position order; thread 0 records how many.
__global__ __launch_bounds__(PR_THREADS) void k_cand_collect(const uint64_t* __restrict__ key,
                                                             int64_t C,
                                                             const int32_t* __restrict__ sel,
                                                             const int32_t* __restrict__ pos,
                                                             int64_t* __restrict__ out,
                                                             pr_state* st, int32_t n_drop) {
  const int64_t t = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
  if (t == 0) st->n_new = min(st->total_ok, n_drop - st->got);
  if (t < C && sel[t]) out[pos[t]] = (int64_t)key[t];
}

// Merge the sorted, disjoint lists acc[0..got) and nw[0..n_new) by rank.
__global__ __launch_bounds__(PR_THREADS) void k_merge_acc(const int64_t* __restrict__ acc,
                                                          const int64_t* __restrict__ nw,
                                                          const pr_state* st,
                                                          int64_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
  const int64_t got = st->got, n_new = st->n_new;
  if (t < got) {
    out[t + lower_bound_i64(nw, n_new, acc[t])] = acc[t];
  } else if (t < got + n_new) {
    const int64_t j = t - got;
    out[j + lower_bound_i64(acc, got, nw[j])] = nw[j];
  }
}

// New COO = survivors + grown positions (value 0), by rank; only once the
// step is complete and clean.
template <typename T>
__global__ __launch_bounds__(PR_THREADS) void k_final_merge(
    const int64_t* __restrict__ surv_lin, const uint32_t* __restrict__ surv_val, int64_t n_surv,
    const int64_t* __restrict__ grown, int64_t n_grown, int32_t K, const pr_state* st,
    int32_t* __restrict__ row, int32_t* __restrict__ col, T* __restrict__ vals,
    int64_t* __restrict__ grown_out) {
  if (st->err || (int64_t)st->got + st->n_new < n_grown) return;
  const int64_t t = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
  int64_t lin, pos;
  uint32_t vb;
  if (t < n_surv) {
    lin = surv_lin[t];
    pos = t + lower_bound_i64(grown, n_grown, lin);
    vb = surv_val[t];
  } else if (t < n_surv + n_grown) {
    const int64_t j = t - n_surv;
    lin = grown[j];
    pos = j + lower_bound_i64(surv_lin, n_surv, lin);
    vb = 0;
    if (grown_out) grown_out[j] = lin;
  } else {
    return;
  }
  row[pos] = (int32_t)(lin / K);
  col[pos] = (int32_t)(lin % K);
  if constexpr (sizeof(T) == 4) {
    ((uint32_t*)vals)[pos] = vb;
  } else {
    vals[pos] = (T)vb;
  }
}

// ================================================================ bitmap plan
// Words of 32 positions (bit b of word w = position 32w + b).

__global__ __launch_bounds__(256) void k_bm_zero(uint4* __restrict__ p, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Support bitmap, a copy of the values, the NaN check and the first select
// histogram (all entries match the empty prefix).  Thread t of a block owns
// entries base + 4t .. base + 4t + 3 (one vector load per array); their
// words and bits go through LDS, and the first entry of each run of equal
// words in the block ORs the run together.  A word wholly inside the block
// is written with a plain store; the (at most two) words a block shares with
// its neighbours are ORed in atomically.  err bits: 1 NaN, 2 index out of
// range, 4 COO not strictly increasing.
template <typename T>
__global__ __launch_bounds__(PR_THREADS) void k_bm_build(
    const int32_t* __restrict__ row, const int32_t* __restrict__ col, const T* __restrict__ vals,
    int64_t nnz, int32_t M, int32_t K, int shift, int32_t vec_ok, pr_state* st,
    uint32_t* __restrict__ sup, T* __restrict__ vals_ws) {
  __shared__ int32_t h[256];
  __shared__ int64_t lw[PR_BLOCK];    // word of each entry (-1: invalid index)
  __shared__ uint32_t lb[PR_BLOCK];   // bit of each entry within its word
  __shared__ int64_t edge[2];         // words of entries base-1 and base+n (-2: none)
  const int t = threadIdx.x;
  h[t] = 0;
  const int64_t base = (int64_t)blockIdx.x * PR_BLOCK;
  const int n = (int)std::min<int64_t>(PR_BLOCK, nnz - base);
  const int64_t k0 = base + 4 * t;
  auto lin_of = [&](int32_t r, int32_t c) -> int64_t {
    return (r < 0 || r >= M || c < 0 || c >= K) ? -1 : (int64_t)r * K + c;
  };
  if (t < 2) {
    const int64_t k = t == 0 ? base - 1 : base + n;
    edge[t] = (k >= 0 && k < nnz) ? lin_of(row[k], col[k]) : -2;
    if (edge[t] >= 0) edge[t] >>= 5;
  }
  int32_t r4[4], c4[4];
  T v4[4];
  if (vec_ok && k0 + 3 < nnz) {
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
  int err = 0;
  uint32_t a[4];
  int64_t lin[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool ok = k0 + j < nnz;
    a[j] = magnitude<T>(raw_bits(v4[j]));
    lin[j] = lin_of(r4[j], c4[j]);
    if (ok) {
      vals_ws[k0 + j] = v4[j];
      if (is_nan_mag<T>(a[j])) err |= 1;
      if (lin[j] < 0) err |= 2;
      lw[4 * t + j] = lin[j] < 0 ? -1 : (lin[j] >> 5);
      lb[4 * t + j] = 1u << (lin[j] & 31);
    }
  }
  __syncthreads();
  // order check against the previous entry (LDS, or the block's left edge)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * t + j;
    if (i >= n || lin[j] < 0) continue;
    int64_t plin;
    if (j > 0) plin = lin[j - 1];
    else if (i > 0) plin = lin_of(row[k0 - 1], col[k0 - 1]);
    else plin = base > 0 ? lin_of(row[base - 1], col[base - 1]) : -1;
    if (plin >= 0 && lin[j] <= plin) err |= 4;
  }
  // runs of equal words: the first entry of each run writes the word
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * t + j;
    if (i >= n) continue;
    const int64_t w = lw[i];
    if (w < 0) continue;
    const bool starts = i == 0 || lw[i - 1] != w;
    if (!starts) continue;
    uint32_t bits = 0;
    int e = i;
    while (e < n && lw[e] == w) bits |= lb[e++];
    const bool shared = (i == 0 && edge[0] == w) || (e == n && edge[1] == w);
    if (shared) atomicOr(&sup[w], bits);
    else sup[w] = bits;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) wave_hist_add(h, (a[j] >> shift) & 255u, k0 + j < nnz);
  if (err) atomicOr(&st->err, err);
  __syncthreads();
  if (h[t]) atomicAdd(&st->hist[0][blockIdx.x % PR_REPL][t], h[t]);
}

// Dropped bitmap: the classify decision of k_pr_apply (same blocks, ties in
// index order), marking dropped positions instead of compacting.
template <typename T>
__global__ __launch_bounds__(PR_THREADS) void k_bm_drop(
    const int32_t* __restrict__ row, const int32_t* __restrict__ col, const T* __restrict__ vals,
    int64_t nnz, int32_t M, int32_t K, const pr_state* st, const int32_t* __restrict__ base_eq,
    uint32_t* __restrict__ dropb) {
  __shared__ int32_t lds[PR_THREADS / SNK_WAVE];
  const uint32_t tau = st->prefix;
  const int32_t need = st->need;
  const int64_t base = (int64_t)blockIdx.x * PR_BLOCK + (int64_t)threadIdx.x * PR_PER_THREAD;
  uint32_t mag[PR_PER_THREAD];
  int32_t eq = 0;
#pragma unroll
  for (int j = 0; j < PR_PER_THREAD; ++j) {
    mag[j] = base + j < nnz ? magnitude<T>(raw_bits(vals[base + j])) : 0u;
    eq += (base + j < nnz && mag[j] == tau);
  }
  int32_t tmp;
  int32_t er = base_eq[blockIdx.x] + block_excl_scan_i32<PR_THREADS>(eq, lds, &tmp);
#pragma unroll
  for (int j = 0; j < PR_PER_THREAD; ++j) {
    const int64_t k = base + j;
    if (k >= nnz) break;
    const bool is_eq = mag[j] == tau;
    const bool drop = mag[j] < tau || (is_eq && er < need);
    er += is_eq;
    if (drop) {
      const int32_t r = row[k], c = col[k];
      if (r < 0 || r >= M || c < 0 || c >= K) continue;
      const int64_t lin = (int64_t)r * K + c;
      atomicOr(&dropb[lin >> 5], 1u << (lin & 31));
    }
  }
}

__device__ __forceinline__ int32_t chunk_taken(const pr_state* st, int slot) {
  int32_t a = 0;
#pragma unroll
  for (int i = 0; i < BM_ACC_REPL; ++i) a += st->ch_acc[slot][i];
  return a;
}

// Regrow chunk c: stream indices [start, start + rem), rem = positions still
// missing, derived from chunk c-1's record.  A candidate is taken if it is
// outside the old support and its bit in the grown bitmap was clear (an
// atomic test-and-set).  Block 0 records the chunk and clears the taken
// count of the next slot.  err bit 8: stream index bound passed.
__global__ __launch_bounds__(PR_THREADS) void k_bm_chunk(int32_t c, uint64_t s, uint64_t MK,
                                                         int32_t n_drop,
                                                         const uint32_t* __restrict__ sup,
                                                         uint32_t* __restrict__ grown,
                                                         pr_state* st) {
  __shared__ int32_t wsum[PR_THREADS / SNK_WAVE];
  const int slot = c & (BM_SLOTS - 1);
  int64_t start = 0;
  int32_t rem = n_drop;
  if (c > 0) {
    const int ps = (c - 1) & (BM_SLOTS - 1);
    start = st->ch_start[ps] + st->ch_rem[ps];
    rem = st->ch_rem[ps] - chunk_taken(st, ps);
  }
  const bool lead = blockIdx.x == 0 && threadIdx.x == 0;
  if (lead) {
    st->ch_start[slot] = start;
    st->ch_rem[slot] = rem;
  }
  if (blockIdx.x == 0 && threadIdx.x < BM_ACC_REPL)
    st->ch_acc[(c + 1) & (BM_SLOTS - 1)][threadIdx.x] = 0;
  if (st->err || rem <= 0) return;
  if (start > (1ll << 40)) {
    if (lead) atomicOr(&st->err, 8);
    return;
  }
  int32_t acc = 0;
  const int64_t end = start + rem;
  for (int64_t i = start + (int64_t)blockIdx.x * PR_THREADS + threadIdx.x; i < end;
       i += (int64_t)gridDim.x * PR_THREADS) {
    const uint64_t p = __umul64hi(sm64_mix(s + ((uint64_t)i + 1) * SM64_GAMMA), MK);
    const uint32_t bit = 1u << (p & 31);
    const int64_t w = (int64_t)(p >> 5);
    if (sup[w] & bit) continue;
    if (!(atomicOr(&grown[w], bit) & bit)) ++acc;
  }
  // one atomic per block, spread over BM_ACC_REPL counters: same-address
  // device atomics serialise (~10 ns each)
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, SNK_WAVE);
  if (lane_id() == 0) wsum[threadIdx.x / SNK_WAVE] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t b = 0;
#pragma unroll
    for (int i = 0; i < PR_THREADS / SNK_WAVE; ++i) b += wsum[i];
    if (b) atomicAdd(&st->ch_acc[slot][blockIdx.x % BM_ACC_REPL], b);
  }
}

constexpr int BM_WPT = 4;                       // bitmap words per thread
constexpr int BM_WPB = BM_WPT * PR_THREADS;     // words per block

__device__ __forceinline__ int4 bm_counts(uint32_t S, uint32_t D, uint32_t G) {
  return make_int4(__popc((S & ~D) | G), __popc(S), __popc(D), __popc(G));
}

// Per block of BM_WPB words: popcounts of (new support, old support,
// dropped, grown).
__global__ __launch_bounds__(PR_THREADS) void k_bm_wsum(const uint32_t* __restrict__ sup,
                                                        const uint32_t* __restrict__ dropb,
                                                        const uint32_t* __restrict__ grown,
                                                        int64_t W, int4* __restrict__ bsum) {
  __shared__ int32_t lds[4][PR_THREADS / SNK_WAVE];
  const int64_t w0 = (int64_t)blockIdx.x * BM_WPB;
  int4 c = make_int4(0, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < BM_WPT; ++j) {
    const int64_t w = w0 + j * PR_THREADS + threadIdx.x;
    if (w < W) {
      const int4 d = bm_counts(sup[w], dropb[w], grown[w]);
      c.x += d.x; c.y += d.y; c.z += d.z; c.w += d.w;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    c.x += __shfl_xor(c.x, off, SNK_WAVE);
    c.y += __shfl_xor(c.y, off, SNK_WAVE);
    c.z += __shfl_xor(c.z, off, SNK_WAVE);
    c.w += __shfl_xor(c.w, off, SNK_WAVE);
  }
  const int wv = threadIdx.x / SNK_WAVE;
  if (lane_id() == 0) {
    lds[0][wv] = c.x; lds[1][wv] = c.y; lds[2][wv] = c.z; lds[3][wv] = c.w;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int4 tot = make_int4(0, 0, 0, 0);
    for (int i = 0; i < PR_THREADS / SNK_WAVE; ++i) {
      tot.x += lds[0][i]; tot.y += lds[1][i]; tot.z += lds[2][i]; tot.w += lds[3][i];
    }
    bsum[blockIdx.x] = tot;
  }
}

// One workgroup: exclusive prefix of n int4 block sums.  Thread t owns a
// contiguous segment: totals, one block scan, then the segment's prefixes.
constexpr int BM_SCAN_THREADS = 1024;
__global__ __launch_bounds__(BM_SCAN_THREADS) void k_bm_bscan(const int4* __restrict__ in,
                                                              int4* __restrict__ out, int64_t n) {
  __shared__ int32_t lds[BM_SCAN_THREADS / SNK_WAVE];
  const int64_t per = cdiv_dev(n, BM_SCAN_THREADS);
  const int64_t a = std::min<int64_t>(n, (int64_t)threadIdx.x * per);
  const int64_t b = std::min<int64_t>(n, a + per);
  int4 s = make_int4(0, 0, 0, 0);
  for (int64_t i = a; i < b; ++i) {
    const int4 v = in[i];
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  int32_t tot;
  int4 e;
  e.x = block_excl_scan_i32<BM_SCAN_THREADS>(s.x, lds, &tot);
  e.y = block_excl_scan_i32<BM_SCAN_THREADS>(s.y, lds, &tot);
  e.z = block_excl_scan_i32<BM_SCAN_THREADS>(s.z, lds, &tot);
  e.w = block_excl_scan_i32<BM_SCAN_THREADS>(s.w, lds, &tot);
  for (int64_t i = a; i < b; ++i) {
    const int4 v = in[i];
    out[i] = e;
    e.x += v.x; e.y += v.y; e.z += v.z; e.w += v.w;
  }
}

// New COO from the words of (support & ~dropped) | grown, in position order;
// a survivor's value is the old value at its rank in the old support.  Also
// the dropped and grown lists.  Does nothing unless chunk `c_last` left no
// position missing and no error was seen.  Writes are clamped to nnz /
// n_drop.
template <typename T>
__global__ __launch_bounds__(PR_THREADS) void k_bm_emit(
    const uint32_t* __restrict__ sup, const uint32_t* __restrict__ dropb,
    const uint32_t* __restrict__ grown, int64_t W, const int4* __restrict__ boff,
    const T* __restrict__ vals_ws, int32_t K, int64_t nnz, int64_t n_drop, const pr_state* st,
    int32_t c_last, int32_t* __restrict__ row, int32_t* __restrict__ col, T* __restrict__ vals,
    int64_t* __restrict__ dropped_lin, int64_t* __restrict__ grown_lin) {
  __shared__ int32_t lds[PR_THREADS / SNK_WAVE];
  const int ls = c_last & (BM_SLOTS - 1);
  if (st->err || st->ch_rem[ls] - chunk_taken(st, ls) > 0) return;
  const int64_t w0 = (int64_t)blockIdx.x * BM_WPB + (int64_t)threadIdx.x * BM_WPT;
  static_assert(BM_WPT == 4, "one uint4 of words per thread");
  uint32_t S[BM_WPT] = {0u, 0u, 0u, 0u}, D[BM_WPT] = {0u, 0u, 0u, 0u}, G[BM_WPT] = {0u, 0u, 0u, 0u};
  if (w0 < W) {  // the bitmaps are zero-padded to a multiple of 4 words
    const uint4 s4 = *reinterpret_cast<const uint4*>(sup + w0);
    const uint4 d4 = *reinterpret_cast<const uint4*>(dropb + w0);
    const uint4 g4 = *reinterpret_cast<const uint4*>(grown + w0);
    S[0] = s4.x; S[1] = s4.y; S[2] = s4.z; S[3] = s4.w;
    D[0] = d4.x; D[1] = d4.y; D[2] = d4.z; D[3] = d4.w;
    G[0] = g4.x; G[1] = g4.y; G[2] = g4.z; G[3] = g4.w;
  }
  int4 c = make_int4(0, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < BM_WPT; ++j) {
    const int4 d = bm_counts(S[j], D[j], G[j]);
    c.x += d.x; c.y += d.y; c.z += d.z; c.w += d.w;
  }
  int32_t tot;
  const int4 bo = boff[blockIdx.x];
  int64_t qf = bo.x + block_excl_scan_i32<PR_THREADS>(c.x, lds, &tot);
  int64_t qs = bo.y + block_excl_scan_i32<PR_THREADS>(c.y, lds, &tot);
  int64_t qd = bo.z + block_excl_scan_i32<PR_THREADS>(c.z, lds, &tot);
  int64_t qg = bo.w + block_excl_scan_i32<PR_THREADS>(c.w, lds, &tot);
#pragma unroll
  for (int j = 0; j < BM_WPT; ++j) {
    const int64_t pw = (w0 + j) * 32;
    uint32_t F = (S[j] & ~D[j]) | G[j];
    if (F) {
      // row and column of the word's first position; the rest step from it
      const int32_t r0 = (int32_t)(pw / K);
      const int32_t c0 = (int32_t)(pw - (int64_t)r0 * K);
      while (F) {
        const int b = __ffs(F) - 1;
        F &= F - 1;
        if (qf < nnz) {
          int32_t r = r0, c = c0 + b;
          while (c >= K) {
            c -= K;
            ++r;
          }
          row[qf] = r;
          col[qf] = c;
          vals[qf] = ((S[j] >> b) & 1u) ? vals_ws[qs + __popc(S[j] & ((1u << b) - 1u))] : (T)0;
        }
        ++qf;
      }
    }
    qs += __popc(S[j]);
    if (dropped_lin) {
      uint32_t Dw = D[j];
      while (Dw) {
        const int b = __ffs(Dw) - 1;
        Dw &= Dw - 1;
        if (qd < n_drop) dropped_lin[qd] = pw + b;
        ++qd;
      }
    }
    if (grown_lin) {
      uint32_t Gw = G[j];
      while (Gw) {
        const int b = __ffs(Gw) - 1;
        Gw &= Gw - 1;
        if (qg < n_drop) grown_lin[qg] = pw + b;
        ++qg;
      }
    }
  }
}

// ------------------------------------------------------------------ layout
struct pr_layout {
  int64_t C, nblk;
  size_t state, cnt_lt, cnt_eq, base_eq, base_drop, sup, surv_lin, surv_val;
  size_t ck0, ck1, cv0, cv1, ok, okr, sel, selpos, acc0, acc1, nw, tmp, total;
};

static int64_t chunk_size(int32_t M, int32_t K, int64_t nnz, int64_t n_drop) {
  const double MK = (double)M * (double)K;
  const double q = (MK - (double)nnz) / MK;
  double want = q > 0 ? (double)n_drop / q * 1.15 + 2048.0 : 2048.0;
  want = std::min(want, std::max(2048.0, 4.0 * MK + 2048.0));
  want = std::min(want, (double)(1ll << 28));
  return (int64_t)want;
}

static pr_layout make_layout(int32_t M, int32_t K, int64_t nnz, int64_t n_drop) {
  pr_layout L{};
  L.C = chunk_size(M, K, nnz, n_drop);
  L.nblk = std::max<int64_t>(1, cdiv(nnz, PR_BLOCK));
  const int64_t n1 = std::max<int64_t>(nnz, 1);
  const int64_t nd = std::max<int64_t>(n_drop, 1);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.state = take(sizeof(pr_state));
  L.cnt_lt = take(4 * (size_t)L.nblk);
  L.cnt_eq = take(4 * (size_t)L.nblk);
  L.base_eq = take(4 * (size_t)L.nblk);
  L.base_drop = take(4 * (size_t)L.nblk);
  L.sup = take(8 * (size_t)n1);
  L.surv_lin = take(8 * (size_t)n1);
  L.surv_val = take(4 * (size_t)n1);
  L.ck0 = take(8 * (size_t)L.C);
  L.ck1 = take(8 * (size_t)L.C);
  L.cv0 = take(4 * (size_t)L.C);
  L.cv1 = take(4 * (size_t)L.C);
  L.ok = take(4 * (size_t)L.C);
  L.okr = take(4 * (size_t)L.C);
  L.sel = take(4 * (size_t)L.C);
  L.selpos = take(4 * (size_t)L.C);
  L.acc0 = take(8 * (size_t)nd);
  L.acc1 = take(8 * (size_t)nd);
  L.nw = take(8 * (size_t)nd);
  L.tmp = take(std::max(radix_tmp_bytes(L.C), scan_tmp_bytes(L.C)));
  L.total = o;
  return L;
}

// Bitmap plan: taken when the support has density <= 1/4 (so every regrow
// chunk takes at least half of what it draws, up to duplicates) and the
// three bitmaps stay within ~16 bytes per entry (+ 4 MB).
static bool bitmap_plan_ok(int32_t M, int32_t K, int64_t nnz) {
  const int64_t MK = (int64_t)M * K;
  const int64_t W = cdiv(MK, 32);
  return 4 * nnz <= MK && W <= 4 * nnz + (1 << 20);
}

struct bm_layout {
  int64_t nblk, W, W4, nb;
  size_t state, cnt_lt, cnt_eq, base_eq, base_drop, sup, dropb, grown, vals, bsum, boff, total;
};

static bm_layout make_bm_layout(int32_t M, int32_t K, int64_t nnz) {
  bm_layout L{};
  L.nblk = std::max<int64_t>(1, cdiv(nnz, PR_BLOCK));
  L.W = cdiv((int64_t)M * K, 32);
  L.W4 = cdiv(L.W, 4) * 4;
  L.nb = std::max<int64_t>(1, cdiv(L.W, BM_WPB));
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.state = take(sizeof(pr_state));
  L.cnt_lt = take(4 * (size_t)L.nblk);
  L.cnt_eq = take(4 * (size_t)L.nblk);
  L.base_eq = take(4 * (size_t)L.nblk);
  L.base_drop = take(4 * (size_t)L.nblk);
  L.sup = take(4 * (size_t)L.W4);  // the three bitmaps are contiguous (one zero fill)
  L.dropb = take(4 * (size_t)L.W4);
  L.grown = take(4 * (size_t)L.W4);
  L.vals = take(4 * (size_t)std::max<int64_t>(nnz, 1));
  L.bsum = take(16 * (size_t)L.nb);
  L.boff = take(16 * (size_t)L.nb);
  L.total = o;
  return L;
}

// SNACK_PRUNE_PATH=sort forces the sort plan (tests run both plans on the
// same inputs).
static bool use_bitmap_plan(int32_t M, int32_t K, int64_t nnz) {
  const char* e = getenv("SNACK_PRUNE_PATH");
  if (e && e[0] == 's') return false;
  return bitmap_plan_ok(M, K, nnz);
}

size_t prune_regrow_ws_bytes(int32_t M, int32_t K, int64_t nnz, int64_t n_drop) {
  size_t b = make_layout(M, K, nnz, n_drop).total;
  if (bitmap_plan_ok(M, K, nnz)) b = std::max(b, make_bm_layout(M, K, nnz).total);
  return b;
}

template <typename T>
static snack_status run_sort(int32_t* row, int32_t* col, T* vals, int32_t M, int32_t K, int64_t nnz,
                        int64_t n_drop, uint64_t seed, uint64_t step, int64_t* dropped_lin,
                        int64_t* grown_lin, char* ws, hipStream_t s) {
  const pr_layout L = make_layout(M, K, nnz, n_drop);
  pr_state* st = (pr_state*)(ws + L.state);
  int32_t* cnt_lt = (int32_t*)(ws + L.cnt_lt);
  int32_t* cnt_eq = (int32_t*)(ws + L.cnt_eq);
  int32_t* base_eq = (int32_t*)(ws + L.base_eq);
  int32_t* base_drop = (int32_t*)(ws + L.base_drop);
  int64_t* sup = (int64_t*)(ws + L.sup);
  int64_t* surv_lin = (int64_t*)(ws + L.surv_lin);
  uint32_t* surv_val = (uint32_t*)(ws + L.surv_val);
  // sorted candidates end in kbuf[0]/vbuf[0]; the generator writes the key
  // buffer the sort's first pass does not write (pass p writes
  // kbuf[(passes-1-p) & 1])
  uint64_t* const kbuf[2] = {(uint64_t*)(ws + L.ck0), (uint64_t*)(ws + L.ck1)};
  int32_t* const vbuf[2] = {(int32_t*)(ws + L.cv0), (int32_t*)(ws + L.cv1)};
  int32_t* ok = (int32_t*)(ws + L.ok);
  int32_t* okr = (int32_t*)(ws + L.okr);
  int32_t* sel = (int32_t*)(ws + L.sel);
  int32_t* selpos = (int32_t*)(ws + L.selpos);
  int64_t* acc[2] = {(int64_t*)(ws + L.acc0), (int64_t*)(ws + L.acc1)};
  int64_t* nw = (int64_t*)(ws + L.nw);
  void* tmp = ws + L.tmp;
  const int64_t C = L.C;

  hipLaunchKernelGGL(k_pr_init, dim3(PR_REPL), dim3(256), 0, s, st, (int32_t)n_drop);
  const unsigned sel_blocks = (unsigned)L.nblk;
  int pass = 0;
  for (int shift = sizeof(T) == 2 ? 8 : 24; shift >= 0; shift -= 8, ++pass) {
    hipLaunchKernelGGL(k_sel_hist<T>, dim3(sel_blocks), dim3(PR_THREADS), 0, s, vals, nnz, shift,
                       pass, st);
    hipLaunchKernelGGL(k_sel_pick, dim3(1), dim3(256), 0, s, st, shift, pass);
  }
  hipLaunchKernelGGL(k_pr_count<T>, dim3((unsigned)L.nblk), dim3(PR_THREADS), 0, s, vals, nnz,
                     st, cnt_lt, cnt_eq);
  hipLaunchKernelGGL(k_pr_decide, dim3(1), dim3(PR_DECIDE_THREADS), 0, s, cnt_lt, cnt_eq, L.nblk,
                     st, base_eq, base_drop);
  hipLaunchKernelGGL(k_pr_apply<T>, dim3((unsigned)L.nblk), dim3(PR_THREADS), 0, s, row, col,
                     vals, nnz, K, st, base_eq, base_drop, sup, surv_lin, surv_val, dropped_lin);
  if (hipGetLastError() != hipSuccess) return SNACK_E_HIP;

  const uint64_t MK = (uint64_t)M * (uint64_t)K;
  int bits = 0;
  while (bits < 64 && ((MK - 1) >> bits) != 0) ++bits;
  const int passes = std::max(1, (bits + 7) / 8);
  uint64_t* cand = kbuf[passes & 1];
  const uint64_t stream = sm64_mix(seed + (step + 1) * SM64_GAMMA);
  const int64_t n_surv = nnz - n_drop;
  int cur = 0;
  uint64_t base = 0;
  for (int chunk = 0;; ++chunk) {
    hipLaunchKernelGGL(k_cand_gen, g1(C), dim3(PR_THREADS), 0, s, cand, C, stream, base, MK, st);
    if (radix_sort_u64(cand, nullptr, kbuf, vbuf, C, bits, tmp, s) != hipSuccess)
      return SNACK_E_HIP;
    hipLaunchKernelGGL(k_cand_ok, g1(C), dim3(PR_THREADS), 0, s, kbuf[0], vbuf[0], C, sup, nnz,
                       acc[cur], st, ok);
    if (exclusive_scan_i32(ok, okr, C, &st->total_ok, tmp, s) != hipSuccess) return SNACK_E_HIP;
    hipLaunchKernelGGL(k_cand_sel, g1(C), dim3(PR_THREADS), 0, s, vbuf[0], C, ok, okr, st,
                       (int32_t)n_drop, sel);
    if (exclusive_scan_i32(sel, selpos, C, nullptr, tmp, s) != hipSuccess) return SNACK_E_HIP;
    // the first chunk has nothing to merge with: collect straight into the list
    int64_t* dst = chunk == 0 ? acc[cur ^ 1] : nw;
    hipLaunchKernelGGL(k_cand_collect, g1(C), dim3(PR_THREADS), 0, s, kbuf[0], C, sel, selpos,
                       dst, st, (int32_t)n_drop);
    if (chunk > 0)
      hipLaunchKernelGGL(k_merge_acc, g1(n_drop), dim3(PR_THREADS), 0, s, acc[cur], nw, st,
                         acc[cur ^ 1]);
    hipLaunchKernelGGL(k_final_merge<T>, g1(nnz), dim3(PR_THREADS), 0, s, surv_lin, surv_val,
                       n_surv, acc[cur ^ 1], n_drop, K, st, row, col, vals, grown_lin);
    if (hipGetLastError() != hipSuccess) return SNACK_E_HIP;
    int32_t hs[3] = {0, 0, 0};  // err, got, n_new
    if (hipMemcpyAsync(hs, &st->err, sizeof(hs), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return SNACK_E_HIP;
    if (hs[0]) return SNACK_E_NAN;
    if ((int64_t)hs[1] + hs[2] >= n_drop) break;
    cur ^= 1;
    base += (uint64_t)C;
    // n_drop <= free positions is checked by the caller, so the stream
    // reaches n_drop acceptances with probability 1; bound it regardless.
    if (base > (1ull << 40)) return SNACK_E_COUNT;
  }
  return SNACK_OK;
}

// Regrow chunks to launch before the first readback: enough that the
// expected remainder n_drop * (1 - q)^c falls below 1/20, q being a lower
// bound on the acceptance rate.
static int32_t planned_chunks(int64_t MK, int64_t nnz, int64_t n_drop) {
  const double q = std::max(0.5, 1.0 - (double)(nnz + n_drop) / (double)MK);
  int32_t c = 1;
  double rem = (double)n_drop;
  while (rem >= 0.05 && c < 16) {
    rem *= 1.0 - q;
    ++c;
  }
  return std::max<int32_t>(2, c);
}

template <typename T>
static snack_status run_bitmap(int32_t* row, int32_t* col, T* vals, int32_t M, int32_t K,
                               int64_t nnz, int64_t n_drop, uint64_t seed, uint64_t step,
                               int64_t* dropped_lin, int64_t* grown_lin, char* ws, hipStream_t s) {
  const bm_layout L = make_bm_layout(M, K, nnz);
  pr_state* st = (pr_state*)(ws + L.state);
  int32_t* cnt_lt = (int32_t*)(ws + L.cnt_lt);
  int32_t* cnt_eq = (int32_t*)(ws + L.cnt_eq);
  int32_t* base_eq = (int32_t*)(ws + L.base_eq);
  int32_t* base_drop = (int32_t*)(ws + L.base_drop);
  uint32_t* sup = (uint32_t*)(ws + L.sup);
  uint32_t* dropb = (uint32_t*)(ws + L.dropb);
  uint32_t* grown = (uint32_t*)(ws + L.grown);
  T* vals_ws = (T*)(ws + L.vals);
  int4* bsum = (int4*)(ws + L.bsum);
  int4* boff = (int4*)(ws + L.boff);
  const uint64_t MK = (uint64_t)M * (uint64_t)K;

  hipLaunchKernelGGL(k_pr_init, dim3(PR_REPL), dim3(256), 0, s, st, (int32_t)n_drop);
  const int64_t n4 = (int64_t)((L.grown - L.sup) / 16) + L.W4 / 4;
  hipLaunchKernelGGL(k_bm_zero, g1(n4), dim3(256), 0, s, (uint4*)sup, n4);
  const int shift0 = sizeof(T) == 2 ? 8 : 24;
  const int32_t vec_ok = ((uintptr_t)row % 16 == 0 && (uintptr_t)col % 16 == 0 &&
                          (uintptr_t)vals % (4 * sizeof(T)) == 0) ? 1 : 0;
  hipLaunchKernelGGL(k_bm_build<T>, dim3((unsigned)L.nblk), dim3(PR_THREADS), 0, s, row, col,
                     vals, nnz, M, K, shift0, vec_ok, st, sup, vals_ws);
  hipLaunchKernelGGL(k_sel_pick, dim3(1), dim3(256), 0, s, st, shift0, 0);
  int pass = 1;
  for (int shift = shift0 - 8; shift >= 0; shift -= 8, ++pass) {
    hipLaunchKernelGGL(k_sel_hist<T>, dim3((unsigned)L.nblk), dim3(PR_THREADS), 0, s, vals, nnz,
                       shift, pass, st);
    hipLaunchKernelGGL(k_sel_pick, dim3(1), dim3(256), 0, s, st, shift, pass);
  }
  hipLaunchKernelGGL(k_pr_count<T>, dim3((unsigned)L.nblk), dim3(PR_THREADS), 0, s, vals, nnz,
                     st, cnt_lt, cnt_eq);
  hipLaunchKernelGGL(k_pr_decide, dim3(1), dim3(PR_DECIDE_THREADS), 0, s, cnt_lt, cnt_eq, L.nblk,
                     st, base_eq, base_drop);
  hipLaunchKernelGGL(k_bm_drop<T>, dim3((unsigned)L.nblk), dim3(PR_THREADS), 0, s, row, col, vals,
                     nnz, M, K, st, base_eq, dropb);
  if (hipGetLastError() != hipSuccess) return SNACK_E_HIP;

  const uint64_t stream = sm64_mix(seed + (step + 1) * SM64_GAMMA);
  const unsigned chunk_blocks =
      (unsigned)std::min<int64_t>(1024, std::max<int64_t>(1, cdiv(n_drop, PR_THREADS)));
  int32_t c = 0;
  int32_t batch = planned_chunks((int64_t)MK, nnz, n_drop);
  for (;;) {
    for (int32_t e = c + batch; c < e; ++c)
      hipLaunchKernelGGL(k_bm_chunk, dim3(chunk_blocks), dim3(PR_THREADS), 0, s, c, stream, MK,
                         (int32_t)n_drop, sup, grown, st);
    hipLaunchKernelGGL(k_bm_wsum, dim3((unsigned)L.nb), dim3(PR_THREADS), 0, s, sup, dropb, grown,
                       L.W, bsum);
    hipLaunchKernelGGL(k_bm_bscan, dim3(1), dim3(BM_SCAN_THREADS), 0, s, bsum, boff, L.nb);
    hipLaunchKernelGGL(k_bm_emit<T>, dim3((unsigned)L.nb), dim3(PR_THREADS), 0, s, sup, dropb,
                       grown, L.W, boff, vals_ws, K, nnz, n_drop, st, c - 1, row, col, vals,
                       dropped_lin, grown_lin);
    if (hipGetLastError() != hipSuccess) return SNACK_E_HIP;
    const int ls = (c - 1) & (BM_SLOTS - 1);
    int32_t err = 0, rem = 0, taken[BM_ACC_REPL];
    if (hipMemcpyAsync(&err, &st->err, sizeof(err), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipMemcpyAsync(&rem, &st->ch_rem[ls], sizeof(rem), hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipMemcpyAsync(taken, &st->ch_acc[ls][0], sizeof(taken), hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return SNACK_E_HIP;
    for (int i = 0; i < BM_ACC_REPL; ++i) rem -= taken[i];
    if (err & 1) return SNACK_E_NAN;
    if (err & 2) return SNACK_E_COO_RANGE;
    if (err & 4) return SNACK_E_COO_ORDER;
    if (err & 8) return SNACK_E_COUNT;
    if (rem <= 0) break;
    batch = 4;
  }
  return SNACK_OK;
}

snack_status prune_regrow(int32_t* row, int32_t* col, void* vals, snack_dtype dt, int32_t M,
                          int32_t K, int64_t nnz, int64_t n_drop, uint64_t seed, uint64_t step,
                          int64_t* dropped_lin, int64_t* grown_lin, void* ws, size_t ws_bytes,
                          hipStream_t s) {
  if (ws_bytes < prune_regrow_ws_bytes(M, K, nnz, n_drop)) return SNACK_E_WORKSPACE;
  if (use_bitmap_plan(M, K, nnz)) {
    if (dt == SNACK_F32)
      return run_bitmap<float>(row, col, (float*)vals, M, K, nnz, n_drop, seed, step,
                               dropped_lin, grown_lin, (char*)ws, s);
    return run_bitmap<bf16>(row, col, (bf16*)vals, M, K, nnz, n_drop, seed, step, dropped_lin,
                            grown_lin, (char*)ws, s);
  }
  if (dt == SNACK_F32)
    return run_sort<float>(row, col, (float*)vals, M, K, nnz, n_drop, seed, step, dropped_lin,
                           grown_lin, (char*)ws, s);
  return run_sort<bf16>(row, col, (bf16*)vals, M, K, nnz, n_drop, seed, step, dropped_lin,
                        grown_lin, (char*)ws, s);
}

}  // namespace snk
