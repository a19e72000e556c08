// internal.h -- host-side launchers shared between the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/snack.h"

namespace snk {

// ---- exclusive prefix sum of int32 (device) --------------------------------
// out[i] = sum_{j<i} in[j]; in == out is allowed.  If total != NULL the sum
// of all n inputs is written there (device int32).  tmp must hold
// scan_tmp_bytes(n) bytes.
size_t scan_tmp_bytes(int64_t n);
hipError_t exclusive_scan_i32(const int32_t* in, int32_t* out, int64_t n, int32_t* total,
                              void* tmp, hipStream_t s);

// ---- stable LSD radix sort of (key, value) pairs ---------------------------
// Sorts n pairs by the low `bits` bits of the key (8 bits per pass, at least
// one pass).  Input (keys_in, vals_in) is read only; vals_in == NULL means
// value = index.  kbuf/vbuf are two buffer pairs of n elements; the sorted
// result always ends in kbuf[0] / vbuf[0].  If gsrc != NULL the last pass
// also writes gout[i] = gsrc[value[i]].  tmp must hold radix_tmp_bytes(n).
size_t radix_tmp_bytes(int64_t n);
hipError_t radix_sort_u32(const uint32_t* keys_in, const int32_t* vals_in, uint32_t* const kbuf[2],
                          int32_t* const vbuf[2], int64_t n, int bits, const int32_t* gsrc,
                          int32_t* gout, void* tmp, hipStream_t s);
hipError_t radix_sort_u64(const uint64_t* keys_in, const int32_t* vals_in, uint64_t* const kbuf[2],
                          int32_t* const vbuf[2], int64_t n, int bits, void* tmp, hipStream_t s);

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Result words of a call that reads a few words back (prepare, the
// restructure).  Kernels store them at `dev`.  With caller-owned pinned,
// device-mapped host memory (snack_plan.host_words) `dev` maps to `host` and
// the host spins on a completion word that a last one-thread kernel stores;
// otherwise `dev` is device scratch and the words come back by one copy and a
// stream sync into `local`.  Nothing here allocates.
constexpr int RESULT_WORDS = 16;
constexpr int RESULT_DONE_SLOT = 15;
struct result_words {
  int32_t* dev = nullptr;    // device address the kernels store to
  int32_t* host = nullptr;   // caller's pinned words, or NULL
  int32_t local[RESULT_WORDS] = {};
  const int32_t* words() const { return host ? host : local; }
};
// Marks words [0, n) as not written (INT32_MIN) before the kernels run.
hipError_t results_begin(result_words& r, int n, hipStream_t s);
// Waits for every kernel queued on s so far; afterwards words() holds the
// values they stored.  Pinned words: spins on a completion token (falling
// back to hipStreamSynchronize after 20 ms).
hipError_t results_wait(result_words& r, int n, hipStream_t s);
// Device address of caller-owned pinned host memory (NULL if it is not).
int32_t* host_words_device(int32_t* host);
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- products (spmm.hip) ----------------------------------------------------
struct seg_view {          // one compressed view of the sparse matrix
  const int32_t* ptr;      // [S+1] segment offsets
  const int32_t* idx;      // [nnz] gathered feature index of each entry
  const int32_t* perm;     // [nnz] value permutation (NULL = identity)
  const int32_t* part_seg; // [P+1]
  const int32_t* part_nz;  // [P+1]
  const int32_t* cut;      // [P+1] 1 if the cut starting tile p lies inside a segment
  int32_t S;               // segments (output features)
  int32_t F;               // gathered features (input features)
  int32_t P;               // tiles
  int32_t has_split;       // any inner cut (some segment spans tiles)
  int32_t tile;            // items per tile of this view
  int64_t nnz;
};

// act_tmp: scratch for the node-major copy of batch-major activations
// (B > 1); >= elem * B * (F + S) + 256 bytes, or NULL when only node-major
// activations are used.
// act: ACT_NONE / ACT_RELU applied to each finished output (ACT_GELU is run
// as launch_act_inplace after the product).
snack_status launch_seg_spmm(const seg_view& v, const void* vals, snack_dtype dt, const void* X,
                             snack_layout lay, int32_t B, void* Y, float* carry, void* act_tmp,
                             hipStream_t s, int32_t act = 0);
snack_status launch_sddmm(const seg_view& v, const void* dY, const void* X, snack_dtype dt,
                          snack_layout lay, int32_t B, void* dV, void* act_tmp, hipStream_t s);
// Column view, B <= 32: dX = dY W, dV (nullable) and, if lr != 0, the
// in-place update vals <- vals - lr * dV, in one pass.
// vals_t (nullable): the values in column order, read coalesced instead of
// through perm, and updated with them when lr != 0.
snack_status launch_bwd_fused(const seg_view& v, void* vals, void* vals_t, snack_dtype dt,
                              const void* X, const void* dY, snack_layout lay, int32_t B,
                              void* dX, void* dV, float lr, float* carry, void* act_tmp,
                              hipStream_t s, float* m_t = nullptr, float* v_t = nullptr,
                              const float* adam = nullptr);
// vals_t[i] = vals[perm[i]] for i < nnz.
hipError_t launch_gather_vals_t(const int32_t* perm, const void* vals, snack_dtype dt,
                                void* vals_t, int64_t nnz, hipStream_t s);
// Wave-per-segment products (wave.hip), for views with no split segment.
// Activations already node-major; launch_wave_sddmm returns false (and
// launches nothing) when one pass of the kernel cannot cover the batch.
// With split = true, views with split segments qualify too: their tile
// pieces go through the carry slots (P x B and P x B fp32) and k_fixup.
bool wave_eligible(const seg_view& v, snack_dtype dt, int32_t B, bool split);
void launch_wave_spmm(const seg_view& v, const void* vals, snack_dtype dt, const void* Xt,
                      int32_t B, void* Y, bool node_out, int32_t act, float* carry,
                      hipStream_t s);
// out[s] = act(sum of the carry slots of split segment s) for every split
// segment (k_fixup, spmm.hip).
void launch_fixup(const seg_view& v, snack_dtype dt, bool node_out, int32_t act,
                  const float* carry, void* Y, int32_t B, hipStream_t s);
bool launch_wave_sddmm(const seg_view& v, const void* dYt, const void* Xt, snack_dtype dt,
                       int32_t B, void* dV, hipStream_t s);
// Column view: dX, dV (nullable) and the optional update (wave_fused.hip).
// With adam (NULL for SGD): the Adam step instead, hyperparameters
// {lr, beta1, beta2, eps, 1/(1-beta1^t), 1/(1-beta2^t)}, moments m_t, v_t
// (fp32, column order).
bool launch_wave_bwd_fused(const seg_view& v, void* vals, void* vals_t, snack_dtype dt,
                           const void* dYt, const void* Xt, int32_t B, void* dX, void* dV,
                           float lr, bool node_out, hipStream_t s, float* m_t = nullptr,
                           float* v_t = nullptr, const float* adam = nullptr);
hipError_t launch_transpose2(snack_dtype dt, const void* in0, void* out0, int32_t R0, int32_t C0,
                             const void* in1, void* out1, int32_t R1, int32_t C1,
                             hipStream_t s);

// ---- prepare (prepare.hip) ----------------------------------------------------
// Flags are per block (errs: seg_bounds_blocks(nnz) ints, splits:
// tiles_blocks(S) ints), written by every block; launch_prepare_result ORs
// them into res[0..2] (pinned host memory).  errs may be NULL (no
// validation).
int64_t seg_bounds_blocks(int64_t nnz);
int64_t tiles_blocks(int32_t S);
hipError_t launch_seg_bounds(const int32_t* keys, const int32_t* col, int64_t nnz, int32_t S,
                             int32_t K, int32_t* ptr, int32_t* errs, hipStream_t s);
hipError_t launch_tiles(const int32_t* ptr, int32_t S, int64_t nnz, int32_t T, int32_t P,
                        int32_t* part_seg, int32_t* part_nz, int32_t* cut, int32_t* splits,
                        hipStream_t s);
hipError_t launch_prepare_result(const int32_t* errs, int64_t n_errs, const int32_t* rsplit,
                                 int64_t n_r, const int32_t* csplit, int64_t n_c, int32_t* res,
                                 hipStream_t s);

// ---- aux kernels (aux.hip) ------------------------------------------------------
// y <- act(y) elementwise over n values of dt (in place).
hipError_t launch_act_inplace(snack_dtype dt, void* y, int64_t n, int32_t act, hipStream_t s);
hipError_t launch_gelu_fwd(const float* z, float* h, int64_t n, hipStream_t s);
hipError_t launch_gelu_bwd(const float* z, const float* dh, float* dz, int64_t n,
                           hipStream_t s);
hipError_t launch_dense_fwd(const void* W, const uint8_t* mask, snack_dtype dt, int32_t M,
                            int32_t K, const void* X, int32_t B, void* Y, hipStream_t s);

// ---- prune / regrow (prune.hip) ---------------------------------------------------
size_t prune_regrow_ws_bytes(int32_t M, int32_t K, int64_t nnz, int64_t n_drop,
                             uint32_t flags);
snack_status prune_regrow(int32_t* row, int32_t* col, void* vals, snack_dtype dt, int32_t M,
                          int32_t K, int64_t nnz, int64_t n_drop, uint64_t seed, uint64_t step,
                          int64_t* dropped_lin, int64_t* grown_lin, void* ws, size_t ws_bytes,
                          uint32_t flags, hipStream_t s);

}  // namespace snk
