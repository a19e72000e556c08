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
// Device plan: a 4-pass (8-bit digit) radix select finds the magnitude of
// the n_drop-th smallest key and how many entries of exactly that magnitude
// are dropped (the first ones in index order, found with a scan); survivors
// are compacted with scans.  Regrowth draws candidates in chunks of C
// stream positions: candidates are radix-sorted by position (stable, so equal
// positions stay in stream order), a candidate is acceptable when it is the
// first occurrence of its position, not in the old support and not taken by
// an earlier chunk (binary searches), and the first `need` acceptable ones in
// stream order are kept (a scan over stream order).  The host reads back one
// counter per chunk.  Finally survivors and grown positions, both sorted,
// are merged by rank.
#include "common.h"
#include "internal.h"

namespace snk {

constexpr int PR_THREADS = 256;

struct pr_state {
  uint32_t prefix;   // radix-select: magnitude bits fixed so far
  uint32_t mask;
  int32_t need;      // drops still to place at the current prefix
  int32_t err;       // 1 = NaN seen
  int32_t got;       // grown positions accepted so far
  int32_t total_ok;  // acceptable candidates in the current chunk
  int32_t n_new;     // positions accepted from the current chunk
  int32_t pad;
  int32_t hist[256];
};

// SplitMix64: state advances by the golden gamma; output = variant-13 mix.
__device__ __forceinline__ uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static inline uint64_t sm64_mix_host(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
constexpr uint64_t SM64_GAMMA = 0x9E3779B97F4A7C15ull;

static inline dim3 g1(int64_t n) {
  return dim3((unsigned)std::max<int64_t>(1, cdiv(n, PR_THREADS)));
}

__global__ void k_pr_state_init(pr_state* st, int32_t n_drop) {
  int t = threadIdx.x;
  st->hist[t] = 0;
  if (t == 0) {
    st->prefix = 0;
    st->mask = 0;
    st->need = n_drop;
    st->err = 0;
    st->got = 0;
    st->total_ok = 0;
    st->n_new = 0;
  }
}

template <typename T>
__global__ __launch_bounds__(PR_THREADS) void k_pr_keys(
    const int32_t* __restrict__ row, const int32_t* __restrict__ col, const T* __restrict__ vals,
    int64_t nnz, int32_t K, uint32_t* __restrict__ mag, int64_t* __restrict__ lin,
    uint32_t* __restrict__ vbits, pr_state* st) {
  int64_t k = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
  if (k >= nnz) return;
  uint32_t b;
  if constexpr (sizeof(T) == 4) b = __float_as_uint(vals[k]);
  else b = (uint32_t)vals[k];
  uint32_t a = sizeof(T) == 2 ? (b & 0x7FFFu) : (b & 0x7FFFFFFFu);
  bool nan = sizeof(T) == 2 ? (a > 0x7F80u) : (a > 0x7F800000u);
  if (nan) atomicOr(&st->err, 1);
  mag[k] = a;
  vbits[k] = b;
  lin[k] = (int64_t)row[k] * K + col[k];
}

__global__ __launch_bounds__(PR_THREADS) void k_sel_hist(const uint32_t* __restrict__ mag,
                                                         int64_t nnz, int shift, pr_state* st) {
  __shared__ int32_t h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  const uint32_t prefix = st->prefix, mask = st->mask;
  for (int64_t k = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x; k < nnz;
       k += (int64_t)gridDim.x * PR_THREADS) {
    uint32_t m = mag[k];
    if ((m & mask) == prefix) atomicAdd(&h[(m >> shift) & 255u], 1);
  }
  __syncthreads();
  if (h[threadIdx.x]) atomicAdd(&st->hist[threadIdx.x], h[threadIdx.x]);
}

__global__ void k_sel_pick(pr_state* st, int shift) {
  if (threadIdx.x != 0) return;
  int32_t need = st->need, cum = 0;
  int d = 0;
  for (; d < 255; ++d) {
    if (cum + st->hist[d] >= need) break;
    cum += st->hist[d];
  }
  st->need = need - cum;
  st->prefix |= (uint32_t)d << shift;
  st->mask |= 255u << shift;
  for (int i = 0; i < 256; ++i) st->hist[i] = 0;
}

__global__ __launch_bounds__(PR_THREADS) void k_pr_eq(const uint32_t* __restrict__ mag,
                                                      int64_t nnz, const pr_state* st,
                                                      int32_t* __restrict__ eq) {
  int64_t k = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
  if (k < nnz) eq[k] = mag[k] == st->prefix ? 1 : 0;
}

// keep[k] = 1 for survivors; drop[k] = 1 for dropped entries.
__global__ __launch_bounds__(PR_THREADS) void k_pr_flags(const uint32_t* __restrict__ mag,
                                                         int64_t nnz, const pr_state* st,
                                                         const int32_t* __restrict__ eq_rank,
                                                         int32_t* __restrict__ keep,
                                                         int32_t* __restrict__ drop) {
  int64_t k = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
  if (k >= nnz) return;
  uint32_t m = mag[k], tau = st->prefix;
  bool d = m < tau || (m == tau && eq_rank[k] < st->need);
  keep[k] = d ? 0 : 1;
  drop[k] = d ? 1 : 0;
}

__global__ __launch_bounds__(PR_THREADS) void k_pr_compact(
    const int64_t* __restrict__ lin, const uint32_t* __restrict__ vbits, int64_t nnz,
    const int32_t* __restrict__ keep, const int32_t* __restrict__ keep_pos,
    const int32_t* __restrict__ drop_pos, int64_t* __restrict__ surv_lin,
    uint32_t* __restrict__ surv_val, int64_t* __restrict__ dropped_lin) {
  int64_t k = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
  if (k >= nnz) return;
  if (keep[k]) {
    surv_lin[keep_pos[k]] = lin[k];
    surv_val[keep_pos[k]] = vbits[k];
  } else if (dropped_lin) {
    dropped_lin[drop_pos[k]] = lin[k];
  }
}

__global__ __launch_bounds__(PR_THREADS) void k_cand_gen(uint64_t* __restrict__ key,
                                                         int32_t* __restrict__ val, int64_t C,
                                                         uint64_t s, uint64_t base,
                                                         uint64_t MK) {
  int64_t t = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
  if (t >= C) return;
  uint64_t i = base + (uint64_t)t;
  uint64_t x = sm64_mix(s + (i + 1) * SM64_GAMMA);
  key[t] = __umul64hi(x, MK);
  val[t] = (int32_t)t;
}

__device__ __forceinline__ bool in_sorted(const int64_t* __restrict__ a, int64_t n, int64_t x) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    int64_t mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo < n && a[lo] == x;
}

__device__ __forceinline__ int64_t lower_bound_i64(const int64_t* __restrict__ a, int64_t n,
                                                   int64_t x) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    int64_t mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// ok_stream[stream index] = candidate acceptable (first occurrence of its
// position, outside the old support and the positions already grown).
__global__ __launch_bounds__(PR_THREADS) void k_cand_ok(
    const uint64_t* __restrict__ key, const int32_t* __restrict__ val, int64_t C,
    const int64_t* __restrict__ sup, int64_t nnz, const int64_t* __restrict__ acc,
    const pr_state* st, int32_t* __restrict__ ok_stream) {
  int64_t t = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
  if (t >= C) return;
  int64_t p = (int64_t)key[t];
  bool first = t == 0 || key[t - 1] != key[t];
  bool ok = first && !in_sorted(sup, nnz, p) && !in_sorted(acc, st->got, p);
  ok_stream[val[t]] = ok ? 1 : 0;
}

__global__ __launch_bounds__(PR_THREADS) void k_cand_sel(const int32_t* __restrict__ val,
                                                         int64_t C,
                                                         const int32_t* __restrict__ ok_stream,
                                                         const int32_t* __restrict__ ok_rank,
                                                         const pr_state* st, int32_t n_drop,
                                                         int32_t* __restrict__ sel) {
  int64_t t = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
  if (t >= C) return;
  int32_t v = val[t];
  sel[t] = (ok_stream[v] && ok_rank[v] < n_drop - st->got) ? 1 : 0;
}

__global__ __launch_bounds__(PR_THREADS) void k_cand_collect(const uint64_t* __restrict__ key,
                                                             int64_t C,
                                                             const int32_t* __restrict__ sel,
                                                             const int32_t* __restrict__ pos,
                                                             int64_t* __restrict__ out) {
  int64_t t = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
  if (t < C && sel[t]) out[pos[t]] = (int64_t)key[t];
}

// Merge the sorted, disjoint lists acc[0..got) and nw[0..n_new) by rank.
__global__ __launch_bounds__(PR_THREADS) void k_merge_acc(const int64_t* __restrict__ acc,
                                                          const int64_t* __restrict__ nw,
                                                          const pr_state* st,
                                                          int64_t* __restrict__ out) {
  int64_t t = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
  const int64_t got = st->got, n_new = st->n_new;
  if (t < got) {
    out[t + lower_bound_i64(nw, n_new, acc[t])] = acc[t];
  } else if (t < got + n_new) {
    int64_t j = t - got;
    out[j + lower_bound_i64(acc, got, nw[j])] = nw[j];
  }
}

__global__ void k_chunk_done(pr_state* st, int32_t n_drop) {
  if (threadIdx.x == 0) {
    int32_t take = min(st->total_ok, n_drop - st->got);
    st->n_new = take;
  }
}

__global__ void k_chunk_commit(pr_state* st) {
  if (threadIdx.x == 0) {
    st->got += st->n_new;
    st->n_new = 0;
  }
}

template <typename T>
__global__ __launch_bounds__(PR_THREADS) void k_final_merge(
    const int64_t* __restrict__ surv_lin, const uint32_t* __restrict__ surv_val, int64_t n_surv,
    const int64_t* __restrict__ grown, int64_t n_grown, int32_t K, int32_t* __restrict__ row,
    int32_t* __restrict__ col, T* __restrict__ vals, int64_t* __restrict__ grown_out) {
  int64_t t = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
  int64_t lin, pos;
  uint32_t vb;
  if (t < n_surv) {
    lin = surv_lin[t];
    pos = t + lower_bound_i64(grown, n_grown, lin);
    vb = surv_val[t];
  } else if (t < n_surv + n_grown) {
    int64_t j = t - n_surv;
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
  int64_t C;
  size_t state, mag, lin, vbits, f_a, f_b, s_a, s_b, surv_lin, surv_val;
  size_t ckey0, ckey1, cval0, cval1, okr, acc0, acc1, nw, tmp, total;
};

static int64_t chunk_size(int32_t M, int32_t K, int64_t nnz, int64_t n_drop) {
  double MK = (double)M * (double)K;
  double q = (MK - (double)nnz) / MK;
  double want = q > 0 ? (double)n_drop / q * 1.15 + 2048.0 : 2048.0;
  double cap = std::max(2048.0, 4.0 * MK + 2048.0);
  want = std::min(want, cap);
  want = std::min(want, (double)(1ll << 28));
  return (int64_t)want;
}

static pr_layout make_layout(int32_t M, int32_t K, int64_t nnz, int64_t n_drop) {
  pr_layout L{};
  L.C = chunk_size(M, K, nnz, n_drop);
  const int64_t n1 = std::max<int64_t>(nnz, 1);
  const int64_t nf = std::max<int64_t>(n1, L.C);
  const int64_t nd = std::max<int64_t>(n_drop, 1);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.state = take(sizeof(pr_state));
  L.mag = take(4 * (size_t)n1);
  L.lin = take(8 * (size_t)n1);
  L.vbits = take(4 * (size_t)n1);
  L.f_a = take(4 * (size_t)nf);
  L.f_b = take(4 * (size_t)n1);
  L.s_a = take(4 * (size_t)nf);
  L.s_b = take(4 * (size_t)n1);
  L.surv_lin = take(8 * (size_t)n1);
  L.surv_val = take(4 * (size_t)n1);
  L.ckey0 = take(8 * (size_t)L.C);
  L.ckey1 = take(8 * (size_t)L.C);
  L.cval0 = take(4 * (size_t)L.C);
  L.cval1 = take(4 * (size_t)L.C);
  L.okr = take(4 * (size_t)L.C);
  L.acc0 = take(8 * (size_t)nd);
  L.acc1 = take(8 * (size_t)nd);
  L.nw = take(8 * (size_t)nd);
  L.tmp = take(std::max(radix_tmp_bytes(L.C), scan_tmp_bytes(nf)));
  L.total = o;
  return L;
}

size_t prune_regrow_ws_bytes(int32_t M, int32_t K, int64_t nnz, int64_t n_drop) {
  return make_layout(M, K, nnz, n_drop).total;
}

template <typename T>
static snack_status run(int32_t* row, int32_t* col, T* vals, int32_t M, int32_t K, int64_t nnz,
                        int64_t n_drop, uint64_t seed, uint64_t step, int64_t* dropped_lin,
                        int64_t* grown_lin, char* ws, hipStream_t s) {
  const pr_layout L = make_layout(M, K, nnz, n_drop);
  pr_state* st = (pr_state*)(ws + L.state);
  uint32_t* mag = (uint32_t*)(ws + L.mag);
  int64_t* lin = (int64_t*)(ws + L.lin);
  uint32_t* vbits = (uint32_t*)(ws + L.vbits);
  int32_t* f_a = (int32_t*)(ws + L.f_a);
  int32_t* f_b = (int32_t*)(ws + L.f_b);
  int32_t* s_a = (int32_t*)(ws + L.s_a);
  int32_t* s_b = (int32_t*)(ws + L.s_b);
  int64_t* surv_lin = (int64_t*)(ws + L.surv_lin);
  uint32_t* surv_val = (uint32_t*)(ws + L.surv_val);
  uint64_t* ck0 = (uint64_t*)(ws + L.ckey0);
  uint64_t* ck1 = (uint64_t*)(ws + L.ckey1);
  int32_t* cv0 = (int32_t*)(ws + L.cval0);
  int32_t* cv1 = (int32_t*)(ws + L.cval1);
  int32_t* okr = (int32_t*)(ws + L.okr);
  int64_t* acc[2] = {(int64_t*)(ws + L.acc0), (int64_t*)(ws + L.acc1)};
  int64_t* nw = (int64_t*)(ws + L.nw);
  void* tmp = ws + L.tmp;
  hipError_t e;

  hipLaunchKernelGGL(k_pr_state_init, dim3(1), dim3(256), 0, s, st, (int32_t)n_drop);
  hipLaunchKernelGGL(k_pr_keys<T>, g1(nnz), dim3(PR_THREADS), 0, s, row, col, vals, nnz, K, mag,
                     lin, vbits, st);
  // radix select of the n_drop-th smallest magnitude (MSB digit first)
  const unsigned sel_blocks = (unsigned)std::min<int64_t>(1024, std::max<int64_t>(1, cdiv(nnz, 4096)));
  for (int shift = 24; shift >= 0; shift -= 8) {
    hipLaunchKernelGGL(k_sel_hist, dim3(sel_blocks), dim3(PR_THREADS), 0, s, mag, nnz, shift, st);
    hipLaunchKernelGGL(k_sel_pick, dim3(1), dim3(64), 0, s, st, shift);
  }
  hipLaunchKernelGGL(k_pr_eq, g1(nnz), dim3(PR_THREADS), 0, s, mag, nnz, st, f_a);
  if ((e = exclusive_scan_i32(f_a, s_a, nnz, nullptr, tmp, s)) != hipSuccess) return SNACK_E_HIP;
  hipLaunchKernelGGL(k_pr_flags, g1(nnz), dim3(PR_THREADS), 0, s, mag, nnz, st, s_a, f_b, f_a);
  if ((e = exclusive_scan_i32(f_b, s_b, nnz, nullptr, tmp, s)) != hipSuccess) return SNACK_E_HIP;
  if ((e = exclusive_scan_i32(f_a, s_a, nnz, nullptr, tmp, s)) != hipSuccess) return SNACK_E_HIP;
  hipLaunchKernelGGL(k_pr_compact, g1(nnz), dim3(PR_THREADS), 0, s, lin, vbits, nnz, f_b, s_b,
                     s_a, surv_lin, surv_val, dropped_lin);
  if (hipGetLastError() != hipSuccess) return SNACK_E_HIP;

  // regrowth
  const uint64_t MK = (uint64_t)M * (uint64_t)K;
  int bits = 0;
  while (bits < 64 && ((MK - 1) >> bits) != 0) ++bits;
  const uint64_t stream = sm64_mix_host(seed + (step + 1) * SM64_GAMMA);
  const int64_t C = L.C;
  int cur = 0;
  uint64_t base = 0;
  int32_t host_state[2] = {0, 0};  // err, got
  for (;;) {
    hipLaunchKernelGGL(k_cand_gen, g1(C), dim3(PR_THREADS), 0, s, ck0, cv0, C, stream, base, MK);
    uint64_t* sk;
    int32_t* sv;
    if ((e = radix_sort_u64(ck0, cv0, ck1, cv1, C, bits, &sk, &sv, tmp, s)) != hipSuccess)
      return SNACK_E_HIP;
    hipLaunchKernelGGL(k_cand_ok, g1(C), dim3(PR_THREADS), 0, s, sk, sv, C, lin, nnz, acc[cur],
                       st, f_a);
    if ((e = exclusive_scan_i32(f_a, okr, C, &st->total_ok, tmp, s)) != hipSuccess)
      return SNACK_E_HIP;
    hipLaunchKernelGGL(k_cand_sel, g1(C), dim3(PR_THREADS), 0, s, sv, C, f_a, okr, st,
                       (int32_t)n_drop, s_a);
    // candidates in position order -> compaction positions
    int32_t* selpos = (sv == cv0) ? cv1 : cv0;  // free int buffer of size C
    if ((e = exclusive_scan_i32(s_a, selpos, C, nullptr, tmp, s)) != hipSuccess)
      return SNACK_E_HIP;
    hipLaunchKernelGGL(k_cand_collect, g1(C), dim3(PR_THREADS), 0, s, sk, C, s_a, selpos, nw);
    hipLaunchKernelGGL(k_chunk_done, dim3(1), dim3(64), 0, s, st, (int32_t)n_drop);
    hipLaunchKernelGGL(k_merge_acc, g1(n_drop), dim3(PR_THREADS), 0, s, acc[cur], nw, st,
                       acc[cur ^ 1]);
    hipLaunchKernelGGL(k_chunk_commit, dim3(1), dim3(64), 0, s, st);
    cur ^= 1;
    if (hipGetLastError() != hipSuccess) return SNACK_E_HIP;
    if (hipMemcpyAsync(host_state, &st->err, sizeof(int32_t) * 2, hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return SNACK_E_HIP;
    if (host_state[0]) return SNACK_E_NAN;
    if (host_state[1] >= n_drop) break;
    base += (uint64_t)C;
    // n_drop <= free positions is checked by the caller, so the stream
    // reaches n_drop acceptances with probability 1; bound it regardless.
    if (base > (1ull << 40)) return SNACK_E_COUNT;
  }
  const int64_t n_surv = nnz - n_drop;
  hipLaunchKernelGGL(k_final_merge<T>, g1(nnz), dim3(PR_THREADS), 0, s, surv_lin, surv_val,
                     n_surv, acc[cur], n_drop, K, row, col, vals, grown_lin);
  if (hipGetLastError() != hipSuccess) return SNACK_E_HIP;
  return SNACK_OK;
}

snack_status prune_regrow(int32_t* row, int32_t* col, void* vals, snack_dtype dt, int32_t M,
                          int32_t K, int64_t nnz, int64_t n_drop, uint64_t seed, uint64_t step,
                          int64_t* dropped_lin, int64_t* grown_lin, void* ws, size_t ws_bytes,
                          hipStream_t s) {
  if (ws_bytes < prune_regrow_ws_bytes(M, K, nnz, n_drop)) return SNACK_E_WORKSPACE;
  if (dt == SNACK_F32)
    return run<float>(row, col, (float*)vals, M, K, nnz, n_drop, seed, step, dropped_lin,
                      grown_lin, (char*)ws, s);
  return run<bf16>(row, col, (bf16*)vals, M, K, nnz, n_drop, seed, step, dropped_lin, grown_lin,
                   (char*)ws, s);
}

}  // namespace snk
