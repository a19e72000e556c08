// api.cpp -- the C ABI declared in include/snack.h: argument checks, arena
// layout, and the launch sequences of the layer's operations.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>

#include "../../include/snack.h"
#include "internal.h"
#include "prune_common.h"

using namespace snk;

namespace {

constexpr int32_t TILE_MIN = 128;
constexpr int32_t TILE_MAX = 2048;
constexpr int64_t TARGET_TILES = 2048;

// Tile size of a view of S segments: the smallest power of two in
// [TILE_MIN, TILE_MAX] giving at most TARGET_TILES tiles.  For batches wider
// than 32 columns it is also at least twice the mean segment length: a
// segment cut by a tile sends its pieces through fp32 carry slots of P x B
// floats each way, which at 1,024 columns cost more than the balance buys on
// a layer without skew (GPT-2 W1's input gradient: 57 -> 43 us unsplit).
// Only segments well above the mean are still cut.
int32_t auto_tile(int64_t S, int64_t nnz, int32_t max_batch) {
  int32_t T = TILE_MIN;
  while (cdiv(S + nnz, T) > TARGET_TILES && T < TILE_MAX) T *= 2;
  if (max_batch > 32)
    while ((int64_t)T * S < 2 * nnz && T < TILE_MAX) T *= 2;
  return T;
}

inline hipStream_t to_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

__global__ void k_copy_i32(const int32_t* __restrict__ src, int32_t* __restrict__ dst,
                           int64_t n) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

// Arena slots past the public derived arrays: the carry slots of tiles that
// end inside a long segment, the radix-sort buffers of the column view, the
// node-major copy of batch-major activations, and one slot holding the small
// scratch of prepare (per-block error / split flags, scan and sort
// temporaries).
constexpr int SLOT_PRIV = 15;

struct priv_layout {
  size_t res, errs, rsplit, csplit, tmp, total;
};

priv_layout priv_of(const snack_plan* p) {
  priv_layout L{};
  int64_t Pm = std::max<int64_t>(std::max(p->P_row, p->P_col), 1);
  int64_t n = std::max<int64_t>(p->nnz, 1);
  size_t o = 0;
  auto take = [&](size_t b) {
    size_t at = o;
    o = align_up(o + b, 256);
    return at;
  };
  L.res = take(4 * RESULT_WORDS);
  L.errs = take(4 * (size_t)seg_bounds_blocks(p->nnz));
  L.rsplit = take(4 * (size_t)tiles_blocks(p->M));
  L.csplit = take(4 * (size_t)tiles_blocks(p->K));
  L.tmp = take(std::max(radix_tmp_bytes(n), scan_tmp_bytes(std::max<int64_t>(Pm, n))));
  L.total = o;
  return L;
}

enum { S_CARRY = 10, S_KEYS_A = 11, S_KEYS_B = 12, S_VALS_B = 13, S_ACT = 14 };

snack_status check_dtype_layout(snack_dtype dt, snack_layout lay) {
  if (dt != SNACK_F32 && dt != SNACK_BF16) return SNACK_E_DTYPE;
  if (lay != SNACK_BATCH_MAJOR && lay != SNACK_NODE_MAJOR) return SNACK_E_LAYOUT;
  return SNACK_OK;
}

seg_view row_view(const snack_plan* p) {
  char* a = (char*)p->arena;
  seg_view v{};
  v.ptr = (const int32_t*)(a + p->off[SNACK_ARR_ROW_PTR]);
  v.idx = p->col;
  v.perm = nullptr;
  v.part_seg = (const int32_t*)(a + p->off[SNACK_ARR_RPART_SEG]);
  v.part_nz = (const int32_t*)(a + p->off[SNACK_ARR_RPART_NZ]);
  v.cut = (const int32_t*)(a + p->off[SNACK_ARR_RCUT]);
  v.S = p->M;
  v.F = p->K;
  v.P = p->P_row;
  v.has_split = p->has_split_row;
  v.tile = p->tile_row;
  v.nnz = p->nnz;
  return v;
}

seg_view col_view(const snack_plan* p) {
  char* a = (char*)p->arena;
  seg_view v{};
  v.ptr = (const int32_t*)(a + p->off[SNACK_ARR_COL_PTR]);
  v.idx = (const int32_t*)(a + p->off[SNACK_ARR_ROW_T]);
  v.perm = (const int32_t*)(a + p->off[SNACK_ARR_PERM]);
  v.part_seg = (const int32_t*)(a + p->off[SNACK_ARR_CPART_SEG]);
  v.part_nz = (const int32_t*)(a + p->off[SNACK_ARR_CPART_NZ]);
  v.cut = (const int32_t*)(a + p->off[SNACK_ARR_CCUT]);
  v.S = p->K;
  v.F = p->M;
  v.P = p->P_col;
  v.has_split = p->has_split_col;
  v.tile = p->tile_col;
  v.nnz = p->nnz;
  return v;
}

void* act_of(const snack_plan* p) {
  if (p->off[S_ACT] == (size_t)-1) return nullptr;
  return (char*)p->arena + p->off[S_ACT];
}

// The result words of a call on this plan: the caller's pinned host words
// when the plan has them (their device address resolved once per buffer),
// else the plan's private device words.
snack_status plan_results(snack_plan* p, result_words& r) {
  if (p->host_words) {
    if (p->host_words_key != p->host_words || !p->host_words_dev) {
      p->host_words_dev = host_words_device(p->host_words);
      p->host_words_key = p->host_words_dev ? p->host_words : nullptr;
      if (!p->host_words_dev) return SNACK_E_WORKSPACE;
    }
    r.host = p->host_words;
    r.dev = p->host_words_dev;
    return SNACK_OK;
  }
  r.host = nullptr;
  r.dev = (int32_t*)((char*)p->arena + p->off[SLOT_PRIV] + priv_of(p).res);
  return SNACK_OK;
}

#ifdef SNACK_DEBUG_CHECKS
// Debug build: before a product runs, every array its kernels take indices
// from is checked on the device, reading each array only within the size the
// plan gives it: offsets start at 0, never decrease and end at nnz; entry
// indices (the COO columns, row_t) and perm lie in range; tile starts lie in
// range and never decrease; cut flags are 0 or 1.  A violation sets a bit of
// *err (one atomic per wave that found one); the product is then not
// launched.  Bits: 1 row offsets, 2 COO column, 4 row tiles, 8 column
// offsets, 16 row_t, 32 perm, 64 column tiles.
struct dbg_arrays {
  const int32_t *rptr, *col, *rseg, *rnz, *rcut, *cptr, *rowt, *perm, *cseg, *cnz, *ccut;
  int64_t M, K, nnz, Pr, Pc;
};

__device__ __forceinline__ int32_t dbg_offsets(const int32_t* ptr, int64_t S, int64_t nnz,
                                               int64_t i) {
  const int32_t v = ptr[i];
  if (v < 0 || v > nnz) return 1;
  if (i == 0 && v != 0) return 1;
  if (i == S && v != nnz) return 1;
  return (i < S && ptr[i + 1] < v) ? 1 : 0;
}

__device__ __forceinline__ int32_t dbg_tiles(const int32_t* seg, const int32_t* nz,
                                             const int32_t* cut, int64_t P, int64_t S,
                                             int64_t nnz, int64_t p) {
  const int32_t a = seg[p], b = nz[p], c = cut[p];
  if (a < 0 || a > S || b < 0 || b > nnz || (c != 0 && c != 1)) return 1;
  return (p < P && (seg[p + 1] < a || nz[p + 1] < b)) ? 1 : 0;
}

__global__ __launch_bounds__(256) void k_debug_check(dbg_arrays d, int32_t* __restrict__ err) {
  const int64_t n_rp = d.M + 1, n_cp = d.K + 1, n_rt = d.Pr + 1, n_ct = d.Pc + 1;
  const int64_t total = n_rp + n_cp + n_rt + n_ct + 3 * d.nnz;
  int32_t bits = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    int64_t j = i;
    if (j < n_rp) { bits |= dbg_offsets(d.rptr, d.M, d.nnz, j); continue; }
    j -= n_rp;
    if (j < n_cp) { bits |= dbg_offsets(d.cptr, d.K, d.nnz, j) << 3; continue; }
    j -= n_cp;
    if (j < n_rt) { bits |= dbg_tiles(d.rseg, d.rnz, d.rcut, d.Pr, d.M, d.nnz, j) << 2; continue; }
    j -= n_rt;
    if (j < n_ct) { bits |= dbg_tiles(d.cseg, d.cnz, d.ccut, d.Pc, d.K, d.nnz, j) << 6; continue; }
    j -= n_ct;
    if (j < d.nnz) { const int32_t c = d.col[j]; bits |= (c < 0 || c >= d.K) ? 2 : 0; continue; }
    j -= d.nnz;
    if (j < d.nnz) { const int32_t r = d.rowt[j]; bits |= (r < 0 || r >= d.M) ? 16 : 0; continue; }
    j -= d.nnz;
    const int32_t q = d.perm[j];
    bits |= (q < 0 || q >= d.nnz) ? 32 : 0;
  }
  for (int off = 32; off > 0; off >>= 1) bits |= __shfl_xor(bits, off, 64);
  if (bits && __lane_id() == 0) atomicOr(err, bits);
}

__global__ void k_debug_clear(int32_t* err) { *err = 0; }

snack_status debug_check_plan(const snack_plan* p, hipStream_t s) {
  char* a = (char*)p->arena;
  auto arr = [&](int which) { return (const int32_t*)(a + p->off[which]); };
  dbg_arrays d{arr(SNACK_ARR_ROW_PTR), p->col, arr(SNACK_ARR_RPART_SEG),
               arr(SNACK_ARR_RPART_NZ), arr(SNACK_ARR_RCUT), arr(SNACK_ARR_COL_PTR),
               arr(SNACK_ARR_ROW_T), arr(SNACK_ARR_PERM), arr(SNACK_ARR_CPART_SEG),
               arr(SNACK_ARR_CPART_NZ), arr(SNACK_ARR_CCUT), p->M, p->K, p->nnz, p->P_row,
               p->P_col};
  if (p->nnz > 0 && !p->col) return SNACK_E_NOT_PREPARED;
  int32_t* err = (int32_t*)(a + p->off[SLOT_PRIV] + priv_of(p).res);
  int32_t h = 0;
  // on the caller's stream, after its earlier work; the debug build waits
  // for the verdict (one stream synchronisation per product call)
  hipLaunchKernelGGL(k_debug_clear, dim3(1), dim3(1), 0, s, err);
  hipLaunchKernelGGL(k_debug_check, dim3(1024), dim3(256), 0, s, d, err);
  if (hipGetLastError() != hipSuccess ||
      hipMemcpyAsync(&h, err, 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return SNACK_E_HIP;
  return h ? SNACK_E_PLAN_CORRUPT : SNACK_OK;
}
#endif

snack_status check_product(const snack_plan* p, const void* a, const void* b, const void* c,
                           snack_dtype dt, snack_layout lay, int32_t B, void* stream) {
  if (!p) return SNACK_E_NULL;
  if (!p->prepared || !p->arena) return SNACK_E_NOT_PREPARED;
  snack_status st = check_dtype_layout(dt, lay);
  if (st) return st;
  if (B < 0 || B > p->max_batch) return SNACK_E_SHAPE;
  if (B > 0 && (!a || !b || !c)) return SNACK_E_NULL;
#ifdef SNACK_DEBUG_CHECKS
  if (B > 0) return debug_check_plan(p, to_stream(stream));
#else
  (void)stream;
#endif
  return SNACK_OK;
}

}  // namespace

extern "C" {

int32_t snack_version(void) { return 200; }
size_t snack_plan_sizeof(void) { return sizeof(snack_plan); }

const char* snack_status_str(snack_status s) {
  switch (s) {
    case SNACK_OK: return "ok";
    case SNACK_E_NULL: return "null pointer argument";
    case SNACK_E_SHAPE: return "shape out of range";
    case SNACK_E_DTYPE: return "unknown dtype";
    case SNACK_E_LAYOUT: return "unknown layout";
    case SNACK_E_COO_RANGE: return "COO index out of range";
    case SNACK_E_COO_ORDER: return "COO not strictly increasing row-major (unsorted or duplicate)";
    case SNACK_E_NAN: return "NaN value";
    case SNACK_E_COUNT: return "drop count exceeds nnz or free positions";
    case SNACK_E_WORKSPACE: return "arena or workspace too small";
    case SNACK_E_OVERFLOW: return "size exceeds int32 index range";
    case SNACK_E_HIP: return "HIP launch or runtime error";
    case SNACK_E_NOT_PREPARED: return "plan not prepared";
    case SNACK_E_PLAN_CORRUPT: return "plan array or COO index out of range (debug build check)";
    default: return "unknown status";
  }
}

snack_status snack_plan_init(snack_plan* plan, int32_t M, int32_t K, int64_t nnz,
                             int32_t max_batch, int32_t tile_items, uint32_t flags) {
  if (!plan) return SNACK_E_NULL;
  if (flags & ~(uint32_t)SNACK_PLAN_NODE_MAJOR_ONLY) return SNACK_E_LAYOUT;
  if (M < 1 || K < 1 || nnz < 0 || max_batch < 1) return SNACK_E_SHAPE;
  if ((double)nnz > (double)M * (double)K) return SNACK_E_SHAPE;
  if (tile_items < 0 || tile_items > TILE_MAX) return SNACK_E_SHAPE;
  if (nnz + std::max(M, K) + 2 * TILE_MAX >= (int64_t)INT32_MAX) return SNACK_E_OVERFLOW;
  std::memset(plan, 0, sizeof(*plan));
  plan->M = M;
  plan->K = K;
  plan->nnz = nnz;
  plan->max_batch = max_batch;
  plan->tile_row = tile_items ? tile_items : auto_tile(M, nnz, max_batch);
  plan->tile_col = tile_items ? tile_items : auto_tile(K, nnz, max_batch);
  plan->P_row = (int32_t)cdiv((int64_t)M + nnz, plan->tile_row);
  plan->P_col = (int32_t)cdiv((int64_t)K + nnz, plan->tile_col);
  const int64_t n = std::max<int64_t>(nnz, 1);
  size_t o = 0;
  auto take = [&](int slot, size_t bytes) {
    plan->off[slot] = o;
    o = align_up(o + bytes, 256);
  };
  take(SNACK_ARR_ROW_PTR, 4 * ((size_t)M + 1));
  take(SNACK_ARR_RPART_SEG, 4 * ((size_t)plan->P_row + 1));
  take(SNACK_ARR_RPART_NZ, 4 * ((size_t)plan->P_row + 1));
  take(SNACK_ARR_RCUT, 4 * ((size_t)plan->P_row + 1));
  take(SNACK_ARR_COL_PTR, 4 * ((size_t)K + 1));
  take(SNACK_ARR_PERM, 4 * (size_t)n);
  take(SNACK_ARR_ROW_T, 4 * (size_t)n);
  take(SNACK_ARR_CPART_SEG, 4 * ((size_t)plan->P_col + 1));
  take(SNACK_ARR_CPART_NZ, 4 * ((size_t)plan->P_col + 1));
  take(SNACK_ARR_CCUT, 4 * ((size_t)plan->P_col + 1));
  take(S_CARRY, 8 * (size_t)std::max(plan->P_row, plan->P_col) * (size_t)max_batch);
  take(S_KEYS_A, 4 * (size_t)n);
  take(S_KEYS_B, 4 * (size_t)n);
  take(S_VALS_B, 4 * (size_t)n);
  if (!(flags & SNACK_PLAN_NODE_MAJOR_ONLY))
    take(S_ACT, 4 * (size_t)max_batch * ((size_t)M + K) + 512);
  else
    plan->off[S_ACT] = (size_t)-1;
  take(SLOT_PRIV, priv_of(plan).total);
  plan->arena_bytes = o;
  return SNACK_OK;
}

snack_status snack_coo_prepare(snack_plan* plan, const int32_t* row, const int32_t* col,
                               void* arena, size_t arena_bytes, void* stream) {
  if (!plan || !arena) return SNACK_E_NULL;
  if (plan->nnz > 0 && (!row || !col)) return SNACK_E_NULL;
  if (plan->M < 1 || plan->arena_bytes == 0) return SNACK_E_SHAPE;
  if (arena_bytes < plan->arena_bytes) return SNACK_E_WORKSPACE;
  hipStream_t s = to_stream(stream);
  plan->prepared = 0;
  plan->row = row;
  plan->col = col;
  plan->arena = arena;
  char* a = (char*)arena;
  const priv_layout L = priv_of(plan);
  char* priv = a + plan->off[SLOT_PRIV];
  int32_t* errs = (int32_t*)(priv + L.errs);
  int32_t* rsplit = (int32_t*)(priv + L.rsplit);
  int32_t* csplit = (int32_t*)(priv + L.csplit);
  void* tmp = priv + L.tmp;
  const int64_t nnz = plan->nnz;
  int32_t* row_ptr = (int32_t*)(a + plan->off[SNACK_ARR_ROW_PTR]);
  int32_t* col_ptr = (int32_t*)(a + plan->off[SNACK_ARR_COL_PTR]);
  int32_t* perm = (int32_t*)(a + plan->off[SNACK_ARR_PERM]);
  int32_t* row_t = (int32_t*)(a + plan->off[SNACK_ARR_ROW_T]);

  result_words rw;
  if (snack_status st = plan_results(plan, rw)) return st;
  if (results_begin(rw, 3, s) != hipSuccess) return SNACK_E_HIP;

  // Every kernel below is safe on an invalid COO (all writes are clamped);
  // the error bits come back once at the end, with the split flags.
  // 1. validation + row offsets, then the row-view tiles
  if (launch_seg_bounds(row, col, nnz, plan->M, plan->K, row_ptr, errs, s) != hipSuccess)
    return SNACK_E_HIP;
  if (launch_tiles(row_ptr, plan->M, nnz, plan->tile_row, plan->P_row,
                   (int32_t*)(a + plan->off[SNACK_ARR_RPART_SEG]),
                   (int32_t*)(a + plan->off[SNACK_ARR_RPART_NZ]),
                   (int32_t*)(a + plan->off[SNACK_ARR_RCUT]), rsplit, s) != hipSuccess)
    return SNACK_E_HIP;
  // 2. column view: stable radix sort of the entry indices by column (the
  //    last pass also gathers row_t = row[perm]), then offsets and tiles
  if (nnz > 0) {
    int bits = 0;
    while (bits < 31 && ((uint32_t)(plan->K - 1) >> bits) != 0) ++bits;
    uint32_t* const kbuf[2] = {(uint32_t*)(a + plan->off[S_KEYS_A]),
                               (uint32_t*)(a + plan->off[S_KEYS_B])};
    int32_t* const vbuf[2] = {perm, (int32_t*)(a + plan->off[S_VALS_B])};
    if (radix_sort_u32((const uint32_t*)col, nullptr, kbuf, vbuf, nnz, bits, row, row_t, tmp,
                       s) != hipSuccess)
      return SNACK_E_HIP;
    if (launch_seg_bounds((const int32_t*)kbuf[0], nullptr, nnz, plan->K, plan->K, col_ptr,
                          nullptr, s) != hipSuccess)
      return SNACK_E_HIP;
  } else if (launch_seg_bounds(col, nullptr, 0, plan->K, plan->K, col_ptr, nullptr, s) !=
             hipSuccess) {
    return SNACK_E_HIP;
  }
  if (launch_tiles(col_ptr, plan->K, nnz, plan->tile_col, plan->P_col,
                   (int32_t*)(a + plan->off[SNACK_ARR_CPART_SEG]),
                   (int32_t*)(a + plan->off[SNACK_ARR_CPART_NZ]),
                   (int32_t*)(a + plan->off[SNACK_ARR_CCUT]), csplit, s) != hipSuccess)
    return SNACK_E_HIP;
  if (launch_prepare_result(errs, seg_bounds_blocks(nnz), rsplit, tiles_blocks(plan->M), csplit,
                            tiles_blocks(plan->K), rw.dev, s) != hipSuccess ||
      results_wait(rw, 3, s) != hipSuccess)
    return SNACK_E_HIP;
  const int32_t* res = rw.words();
  if (res[0] == INT32_MIN) return SNACK_E_HIP;
  if (res[0] & 1) return SNACK_E_COO_RANGE;
  if (res[0] & 2) return SNACK_E_COO_ORDER;
  plan->has_split_row = res[1] ? 1 : 0;
  plan->has_split_col = res[2] ? 1 : 0;
  plan->prepared = 1;
  return SNACK_OK;
}

const void* snack_plan_array(const snack_plan* plan, int32_t which, int64_t* count) {
  if (!plan || !plan->prepared || which < 0 || which >= SNACK_ARR_COUNT_) return nullptr;
  int64_t n = 0;
  switch (which) {
    case SNACK_ARR_ROW_PTR: n = (int64_t)plan->M + 1; break;
    case SNACK_ARR_RPART_SEG:
    case SNACK_ARR_RPART_NZ: n = (int64_t)plan->P_row + 1; break;
    case SNACK_ARR_RCUT: n = (int64_t)plan->P_row + 1; break;
    case SNACK_ARR_COL_PTR: n = (int64_t)plan->K + 1; break;
    case SNACK_ARR_PERM:
    case SNACK_ARR_ROW_T: n = plan->nnz; break;
    case SNACK_ARR_CPART_SEG:
    case SNACK_ARR_CPART_NZ: n = (int64_t)plan->P_col + 1; break;
    case SNACK_ARR_CCUT: n = (int64_t)plan->P_col + 1; break;
  }
  if (count) *count = n;
  return (const char*)plan->arena + plan->off[which];
}

snack_status snack_spmm_fwd(const snack_plan* plan, const void* vals, snack_dtype dtype,
                            const void* X, snack_layout layout, int32_t B, void* Y,
                            void* stream) {
  snack_status st = check_product(plan, X, Y, plan && plan->nnz ? vals : Y,
                                  dtype, layout, B, stream);
  if (st) return st;
  float* carry = (float*)((char*)plan->arena + plan->off[S_CARRY]);
  return launch_seg_spmm(row_view(plan), vals, dtype, X, layout, B, Y, carry, act_of(plan),
                         to_stream(stream));
}

snack_status snack_spmm_fwd_act(const snack_plan* plan, const void* vals, snack_dtype dtype,
                                const void* X, snack_layout layout, int32_t B, void* Y,
                                int32_t act, void* stream) {
  if (act < SNACK_ACT_NONE || act > SNACK_ACT_GELU) return SNACK_E_SHAPE;
  snack_status st = check_product(plan, X, Y, plan && plan->nnz ? vals : Y,
                                  dtype, layout, B, stream);
  if (st) return st;
  float* carry = (float*)((char*)plan->arena + plan->off[S_CARRY]);
  hipStream_t s = to_stream(stream);
  // ReLU is applied in the product's store; GELU (an erf) runs as one
  // elementwise pass over Y right after, which measured faster than in the
  // product's epilogue
  st = launch_seg_spmm(row_view(plan), vals, dtype, X, layout, B, Y, carry, act_of(plan), s,
                       act == SNACK_ACT_RELU ? SNACK_ACT_RELU : SNACK_ACT_NONE);
  if (st || act != SNACK_ACT_GELU) return st;
  return launch_act_inplace(dtype, Y, (int64_t)B * plan->M, SNACK_ACT_GELU, s) == hipSuccess
             ? SNACK_OK
             : SNACK_E_HIP;
}

snack_status snack_graph_propagate(const snack_plan* plan, const void* vals, snack_dtype dtype,
                                   const void* X, snack_layout layout, int32_t B, int32_t layers,
                                   int32_t act, void* Y, void* tmp, void* stream) {
  if (!plan) return SNACK_E_NULL;
  if (layers < 1 || act < SNACK_ACT_NONE || act > SNACK_ACT_GELU) return SNACK_E_SHAPE;
  if (layers > 1 && plan->M != plan->K) return SNACK_E_SHAPE;
  if (layers > 1 && !tmp) return SNACK_E_NULL;
  if (Y && (Y == X || Y == tmp)) return SNACK_E_SHAPE;
  // layer l writes Y when layers-1-l is even, else tmp, so the last one
  // lands in Y; each reads the previous layer's output
  const void* in = X;
  for (int32_t l = 0; l < layers; ++l) {
    void* out = ((layers - 1 - l) % 2 == 0) ? Y : tmp;
    const snack_status st = snack_spmm_fwd_act(plan, vals, dtype, in, layout, B, out, act, stream);
    if (st) return st;
    in = out;
  }
  return SNACK_OK;
}

snack_status snack_conv1x1(const snack_plan* plan, const void* vals, snack_dtype dtype,
                           const void* X, int32_t N, int32_t HW, int32_t layout, void* Y,
                           void* stream) {
  if (!plan) return SNACK_E_NULL;
  if (layout != SNACK_CONV_NHWC && layout != SNACK_CONV_NCHW) return SNACK_E_LAYOUT;
  if (N < 0 || HW < 0) return SNACK_E_SHAPE;
  if (layout == SNACK_CONV_NHWC) {
    const int64_t B = (int64_t)N * HW;
    if (B > INT32_MAX) return SNACK_E_OVERFLOW;
    return snack_spmm_fwd(plan, vals, dtype, X, SNACK_BATCH_MAJOR, (int32_t)B, Y, stream);
  }
  const size_t es = dtype == SNACK_F32 ? 4 : 2;
  for (int32_t n = 0; n < N; ++n) {
    const snack_status st = snack_spmm_fwd(
        plan, vals, dtype, (const char*)X + (size_t)n * plan->K * HW * es, SNACK_NODE_MAJOR, HW,
        (char*)Y + (size_t)n * plan->M * HW * es, stream);
    if (st) return st;
  }
  return SNACK_OK;
}

snack_status snack_spmm_bwd_input(const snack_plan* plan, const void* vals, snack_dtype dtype,
                                  const void* dY, snack_layout layout, int32_t B, void* dX,
                                  void* stream) {
  snack_status st = check_product(plan, dY, dX, plan && plan->nnz ? vals : dX,
                                  dtype, layout, B, stream);
  if (st) return st;
  float* carry = (float*)((char*)plan->arena + plan->off[S_CARRY]);
  return launch_seg_spmm(col_view(plan), vals, dtype, dY, layout, B, dX, carry, act_of(plan),
                         to_stream(stream));
}

snack_status snack_gather_vals_t(const snack_plan* plan, const void* vals, snack_dtype dtype,
                                 void* vals_t, void* stream) {
  if (!plan) return SNACK_E_NULL;
  if (!plan->prepared || !plan->arena) return SNACK_E_NOT_PREPARED;
  if (dtype != SNACK_F32 && dtype != SNACK_BF16) return SNACK_E_DTYPE;
  if (plan->nnz == 0) return SNACK_OK;
  if (!vals || !vals_t) return SNACK_E_NULL;
  return launch_gather_vals_t(col_view(plan).perm, vals, dtype, vals_t, plan->nnz,
                              to_stream(stream)) == hipSuccess
             ? SNACK_OK
             : SNACK_E_HIP;
}

snack_status snack_spmm_bwd_input_t(const snack_plan* plan, const void* vals_t,
                                    snack_dtype dtype, const void* dY, snack_layout layout,
                                    int32_t B, void* dX, void* stream) {
  snack_status st =
      check_product(plan, dY, dX, plan && plan->nnz ? vals_t : dX, dtype, layout, B, stream);
  if (st) return st;
  float* carry = (float*)((char*)plan->arena + plan->off[S_CARRY]);
  seg_view v = col_view(plan);
  v.perm = nullptr;  // the values arrive in column order
  return launch_seg_spmm(v, vals_t, dtype, dY, layout, B, dX, carry, act_of(plan),
                         to_stream(stream));
}

snack_status snack_sddmm_grad_vals(const snack_plan* plan, const void* dY, const void* X,
                                   snack_dtype dtype, snack_layout layout, int32_t B,
                                   void* dvals, void* stream) {
  snack_status st = check_product(plan, dY, X, plan && plan->nnz ? dvals : X,
                                  dtype, layout, B, stream);
  if (st) return st;
  if (plan->nnz > 0 && !dvals) return SNACK_E_NULL;
  return launch_sddmm(row_view(plan), dY, X, dtype, layout, B, dvals, act_of(plan),
                      to_stream(stream));
}

snack_status snack_spmm_bwd_fused(const snack_plan* plan, void* vals, void* vals_t,
                                  snack_dtype dtype, const void* X, const void* dY,
                                  snack_layout layout, int32_t B, void* dX, void* dvals,
                                  float lr, void* stream) {
  snack_status st = check_product(plan, dY, dX, plan && plan->nnz ? vals : dX,
                                  dtype, layout, B, stream);
  if (st) return st;
  if (B > 0 && !X) return SNACK_E_NULL;
  if (B > 32) return SNACK_E_SHAPE;
  if (!(lr == lr) || lr - lr != 0.f) return SNACK_E_NAN;  // NaN or infinite step size
  float* carry = (float*)((char*)plan->arena + plan->off[S_CARRY]);
  return launch_bwd_fused(col_view(plan), vals, plan->nnz > 0 ? vals_t : nullptr, dtype, X, dY,
                          layout, B, dX, plan->nnz > 0 ? dvals : nullptr, lr, carry,
                          act_of(plan), to_stream(stream));
}

snack_status snack_spmm_bwd_fused_adam(const snack_plan* plan, void* vals, void* vals_t,
                                       snack_dtype dtype, const void* X, const void* dY,
                                       snack_layout layout, int32_t B, void* dX, void* dvals,
                                       float* m_t, float* v_t, const snack_adam* adam,
                                       void* stream) {
  snack_status st = check_product(plan, dY, dX, plan && plan->nnz ? vals : dX,
                                  dtype, layout, B, stream);
  if (st) return st;
  if (!adam || !X) return SNACK_E_NULL;
  if (plan->nnz > 0 && (!m_t || !v_t)) return SNACK_E_NULL;
  if (B < 1 || B > 32 || adam->step < 1) return SNACK_E_SHAPE;
  const float hp[4] = {adam->lr, adam->beta1, adam->beta2, adam->eps};
  for (float x : hp)
    if (!(x == x) || x - x != 0.f) return SNACK_E_NAN;
  if (!(adam->beta1 >= 0.f && adam->beta1 < 1.f && adam->beta2 >= 0.f && adam->beta2 < 1.f &&
        adam->eps >= 0.f))
    return SNACK_E_SHAPE;
  if (plan->nnz == 0) return SNACK_OK;
  // bias corrections in double on the host
  const double c1 = 1.0 / (1.0 - std::pow((double)adam->beta1, (double)adam->step));
  const double c2 = 1.0 / (1.0 - std::pow((double)adam->beta2, (double)adam->step));
  const float h[6] = {adam->lr, adam->beta1, adam->beta2, adam->eps, (float)c1, (float)c2};
  float* carry = (float*)((char*)plan->arena + plan->off[S_CARRY]);
  return launch_bwd_fused(col_view(plan), vals, vals_t, dtype, X, dY, layout, B, dX, dvals, 0.f,
                          carry, act_of(plan), to_stream(stream), m_t, v_t, h);
}

int64_t snack_drop_count(int64_t nnz, int32_t frac_ppm) {
  if (nnz < 0 || frac_ppm < 0) return -1;
  return (int64_t)(((__int128)nnz * frac_ppm + 500000) / 1000000);
}

snack_status snack_prune_regrow_workspace_ex(int32_t M, int32_t K, int64_t nnz, int64_t n_drop,
                                             uint32_t flags, size_t* bytes) {
  if (!bytes) return SNACK_E_NULL;
  if (flags & ~(uint32_t)SNACK_PRUNE_SORT_PLAN) return SNACK_E_LAYOUT;
  if (M < 1 || K < 1 || nnz < 0 || (double)nnz > (double)M * K || n_drop < 0)
    return SNACK_E_SHAPE;
  if (nnz >= (int64_t)INT32_MAX) return SNACK_E_OVERFLOW;
  *bytes = prune_regrow_ws_bytes(M, K, nnz, n_drop, flags);
  return SNACK_OK;
}

snack_status snack_prune_regrow_workspace(int32_t M, int32_t K, int64_t nnz, int64_t n_drop,
                                          size_t* bytes) {
  return snack_prune_regrow_workspace_ex(M, K, nnz, n_drop, 0, bytes);
}

snack_status snack_memory_footprint(int32_t M, int32_t K, int64_t nnz, int32_t max_batch,
                                    snack_dtype dtype, int64_t n_drop, uint32_t plan_flags,
                                    snack_footprint* out) {
  if (!out) return SNACK_E_NULL;
  if (dtype != SNACK_F32 && dtype != SNACK_BF16) return SNACK_E_DTYPE;
  snack_plan plan;
  const snack_status st = snack_plan_init(&plan, M, K, nnz, max_batch, 0, plan_flags);
  if (st != SNACK_OK) return st;
  if (n_drop < 0) return SNACK_E_SHAPE;
  if (n_drop > nnz || n_drop > (int64_t)M * K - nnz) return SNACK_E_COUNT;
  size_t ws = 0;
  if (n_drop > 0) {
    const snack_status sw = snack_prune_regrow_workspace(M, K, nnz, n_drop, &ws);
    if (sw != SNACK_OK) return sw;
  }
  const uint64_t s = dtype == SNACK_F32 ? 4 : 2;
  const uint64_t mk = (uint64_t)M * (uint64_t)K;
  snack_footprint f;
  f.coo = (uint64_t)nnz * (8 + s);
  f.value_grad = (uint64_t)nnz * s;
  f.col_values = (uint64_t)nnz * s;
  f.derived = plan.off[S_CARRY];  // the derived arrays come first in the arena
  f.plan_scratch = plan.arena_bytes - f.derived;
  f.restructure_ws = ws;
  f.sparse_total =
      f.coo + f.value_grad + f.col_values + f.derived + f.plan_scratch + f.restructure_ws;
  f.dense_weight = mk * s;
  f.dense_grad = mk * s;
  f.dense_total = f.dense_weight + f.dense_grad;
  f.mask = mk;
  f.masked_total = f.dense_total + f.mask;
  f.activations = 2 * (uint64_t)max_batch * ((uint64_t)M + (uint64_t)K) * s;
  *out = f;
  return SNACK_OK;
}

snack_status snack_prune_regrow_ex(int32_t* row, int32_t* col, void* vals, snack_dtype dtype,
                                   int32_t M, int32_t K, int64_t nnz, int64_t n_drop,
                                   uint64_t seed, uint64_t step, int64_t* dropped_lin,
                                   int64_t* grown_lin, void* ws, size_t ws_bytes, uint32_t flags,
                                   void* stream) {
  if (dtype != SNACK_F32 && dtype != SNACK_BF16) return SNACK_E_DTYPE;
  if (flags & ~(uint32_t)SNACK_PRUNE_SORT_PLAN) return SNACK_E_LAYOUT;
  if (M < 1 || K < 1 || nnz < 0 || (double)nnz > (double)M * K || n_drop < 0)
    return SNACK_E_SHAPE;
  if (nnz >= (int64_t)INT32_MAX) return SNACK_E_OVERFLOW;
  if (n_drop > nnz || n_drop > (int64_t)M * K - nnz) return SNACK_E_COUNT;
  if (n_drop == 0) return SNACK_OK;
  if (!row || !col || !vals || !ws) return SNACK_E_NULL;
  return prune_regrow(row, col, vals, dtype, M, K, nnz, n_drop, seed, step, dropped_lin,
                      grown_lin, ws, ws_bytes, flags, to_stream(stream));
}

snack_status snack_prune_regrow(int32_t* row, int32_t* col, void* vals, snack_dtype dtype,
                                int32_t M, int32_t K, int64_t nnz, int64_t n_drop,
                                uint64_t seed, uint64_t step, int64_t* dropped_lin,
                                int64_t* grown_lin, void* ws, size_t ws_bytes, void* stream) {
  return snack_prune_regrow_ex(row, col, vals, dtype, M, K, nnz, n_drop, seed, step,
                               dropped_lin, grown_lin, ws, ws_bytes, 0, stream);
}

snack_status snack_prune_regrow_prepared(snack_plan* plan, int32_t* row, int32_t* col,
                                         void* vals, void* vals_t, snack_dtype dtype,
                                         int64_t n_drop, uint64_t seed, uint64_t step,
                                         int64_t* dropped_lin, int64_t* grown_lin, void* ws,
                                         size_t ws_bytes, uint32_t flags, void* stream) {
  if (!plan) return SNACK_E_NULL;
  if (!plan->arena || plan->arena_bytes == 0) return SNACK_E_NOT_PREPARED;
  if (dtype != SNACK_F32 && dtype != SNACK_BF16) return SNACK_E_DTYPE;
  if (flags & ~(uint32_t)SNACK_PRUNE_SORT_PLAN) return SNACK_E_LAYOUT;
  const int32_t M = plan->M, K = plan->K;
  const int64_t nnz = plan->nnz;
  if (n_drop < 0) return SNACK_E_SHAPE;
  if (n_drop > nnz || n_drop > (int64_t)M * K - nnz) return SNACK_E_COUNT;
  if (nnz > 0 && (!row || !col || !vals)) return SNACK_E_NULL;
  hipStream_t s = to_stream(stream);
  // the values in the new column order, after a restructure that did not
  // write them itself
  auto finish_vals_t = [&](snack_status st) {
    if (st != SNACK_OK || !vals_t || nnz == 0) return st;
    return launch_gather_vals_t(col_view(plan).perm, vals, dtype, vals_t, nnz, s) == hipSuccess
               ? SNACK_OK
               : SNACK_E_HIP;
  };
  if (n_drop == 0)
    return finish_vals_t(
        snack_coo_prepare(plan, row, col, plan->arena, plan->arena_bytes, stream));
  if (!ws) return SNACK_E_NULL;
  if (ws_bytes < prune_regrow_ws_bytes(M, K, nnz, n_drop, flags)) return SNACK_E_WORKSPACE;
  if (use_bitmap_plan(M, K, nnz, flags) && prune_bitmap_fused_ok(M, K, nnz)) {
    result_words rw;
    if (snack_status st = plan_results(plan, rw)) return st;
    return prune_bitmap_prepared(plan, row, col, vals, vals_t, dtype, n_drop, seed, step,
                                 dropped_lin, grown_lin, ws, rw, s);
  }
  plan->prepared = 0;
  const snack_status st = prune_regrow(row, col, vals, dtype, M, K, nnz, n_drop, seed, step,
                                       dropped_lin, grown_lin, ws, ws_bytes, flags, s);
  if (st != SNACK_OK) return st;
  return finish_vals_t(snack_coo_prepare(plan, row, col, plan->arena, plan->arena_bytes, stream));
}

snack_status snack_gelu_fwd(const float* z, float* h, int64_t n, void* stream) {
  if (n < 0) return SNACK_E_SHAPE;
  if (n > 0 && (!z || !h)) return SNACK_E_NULL;
  return launch_gelu_fwd(z, h, n, to_stream(stream)) == hipSuccess ? SNACK_OK : SNACK_E_HIP;
}

snack_status snack_gelu_bwd(const float* z, const float* dh, float* dz, int64_t n,
                            void* stream) {
  if (n < 0) return SNACK_E_SHAPE;
  if (n > 0 && (!z || !dh || !dz)) return SNACK_E_NULL;
  return launch_gelu_bwd(z, dh, dz, n, to_stream(stream)) == hipSuccess ? SNACK_OK : SNACK_E_HIP;
}

snack_status snack_dense_fwd(const void* W, const uint8_t* mask, snack_dtype dtype, int32_t M,
                             int32_t K, const void* X, int32_t B, void* Y, void* stream) {
  if (dtype != SNACK_F32 && dtype != SNACK_BF16) return SNACK_E_DTYPE;
  if (M < 1 || K < 1 || B < 0) return SNACK_E_SHAPE;
  if (B > 0 && (!W || !X || !Y)) return SNACK_E_NULL;
  return launch_dense_fwd(W, mask, dtype, M, K, X, B, Y, to_stream(stream)) == hipSuccess
             ? SNACK_OK
             : SNACK_E_HIP;
}

}  // extern "C"
