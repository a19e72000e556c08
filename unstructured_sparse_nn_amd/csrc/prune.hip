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
// Two device plans give identical results.  The bitmap plan
// (prune_bitmap.hip) serves layers of density <= 1/4 with a modest M*K
// grid; this file holds the plan for everything else and the dispatch:
//   select    radix select of the n_drop-th smallest magnitude, per 8-bit
//             digit (2 passes for bf16, 4 for fp32): blocks build local
//             histograms and add them into replicated global ones, then one
//             workgroup sums them and picks the digit (a block scan);
//   classify  per 1024-entry block: count entries below / at the threshold;
//             one workgroup turns the counts into block offsets (ties at the
//             threshold are dropped in index order); a third kernel writes
//             the survivors, the dropped list and the old support;
//   regrow    candidates are drawn C stream positions at a time and radix
//             sorted by position (stable: equal positions keep stream
//             order); a candidate is acceptable if it is the first
//             occurrence of its position and lies outside the old support
//             and the positions taken by earlier chunks (binary searches);
//             the first `need` acceptable ones in stream order are kept (a
//             scan over stream order) and compacted in position order (a
//             scan over sorted order);
//   merge     survivors and grown positions, both sorted, are merged by rank
//             straight into row/col/vals.  It is launched before the
//             readback and does nothing unless the step is complete and no
//             NaN was seen, so the COO is untouched on error.
#include <cstdlib>

#include "common.h"
#include "internal.h"
#include "prune_common.h"

namespace snk {

constexpr int PR_THREADS = 256;
constexpr int PR_PER_THREAD = 4;
constexpr int PR_BLOCK = PR_THREADS * PR_PER_THREAD;  // entries per classify block
constexpr int PR_REPL = 64;

struct pr_state {
  uint32_t prefix;   // radix-select: magnitude bits fixed so far
  uint32_t mask;
  int32_t need;      // drops still to place among entries matching prefix
  int32_t err;       // 1 = NaN seen
  int32_t got;       // grown positions accepted by committed chunks
  int32_t n_new;     // positions accepted by the latest chunk
  int32_t total_ok;  // acceptable candidates in the latest chunk
  int32_t pad;
  // select histograms, spread over PR_REPL replicas (block b adds into
  // replica b % PR_REPL) so that skewed digits do not serialise on a few
  // global atomics
  int32_t hist[4][PR_REPL][256];
};

static inline dim3 g1(int64_t n) {
  return dim3((unsigned)std::max<int64_t>(1, cdiv(n, PR_THREADS)));
}

// grid: PR_REPL blocks of 256 threads
__global__ void k_pr_init(pr_state* st, int32_t n_drop) {
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < 4; ++p) st->hist[p][blockIdx.x][t] = 0;
  if (blockIdx.x != 0) return;
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
  key[t] = sm64_position(s, i, MK);
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

// SNACK_PRUNE_SORT_PLAN forces the sort plan (tests run both plans on the
// same inputs).
bool use_bitmap_plan(int32_t M, int32_t K, int64_t nnz, uint32_t flags) {
  if (flags & SNACK_PRUNE_SORT_PLAN) return false;
  return prune_bitmap_ok(M, K, nnz);
}

// The workspace of the plan that will run (the same choice as the calls).
size_t prune_regrow_ws_bytes(int32_t M, int32_t K, int64_t nnz, int64_t n_drop,
                             uint32_t flags) {
  if (use_bitmap_plan(M, K, nnz, flags)) return prune_bitmap_ws_bytes(M, K, nnz);
  return make_layout(M, K, nnz, n_drop).total;
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

snack_status prune_regrow(int32_t* row, int32_t* col, void* vals, snack_dtype dt, int32_t M,
                          int32_t K, int64_t nnz, int64_t n_drop, uint64_t seed, uint64_t step,
                          int64_t* dropped_lin, int64_t* grown_lin, void* ws, size_t ws_bytes,
                          uint32_t flags, hipStream_t s) {
  if (ws_bytes < prune_regrow_ws_bytes(M, K, nnz, n_drop, flags)) return SNACK_E_WORKSPACE;
  if (use_bitmap_plan(M, K, nnz, flags))
    return prune_bitmap(row, col, vals, dt, M, K, nnz, n_drop, seed, step, dropped_lin, grown_lin,
                        ws, s);
  if (dt == SNACK_F32)
    return run_sort<float>(row, col, (float*)vals, M, K, nnz, n_drop, seed, step, dropped_lin,
                           grown_lin, (char*)ws, s);
  return run_sort<bf16>(row, col, (bf16*)vals, M, K, nnz, n_drop, seed, step, dropped_lin,
                        grown_lin, (char*)ws, s);
}

}  // namespace snk
