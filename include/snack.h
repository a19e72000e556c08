/*
 * snack.h -- C ABI of a truly sparse linear layer for AMD Instinct MI355X
 * (gfx950).
 *
 * The layer follows "Beyond Masked Sparsity: SNACK Enables Truly Sparse
 * Neural Networks on GPU" (Abstract): the weight W (M x K, out x in) is kept
 * only as its nonzero connections in COO form (row, col, value), forward and
 * backward products touch only those nonzeros, and connections can be
 * restructured (dynamic sparse training).  The page gives the operations in
 * words; their exact forms are stated below with each entry point.
 *
 * Conventions shared by every entry point
 *   - COO: row[k], col[k] are int32 device arrays of length nnz, strictly
 *     increasing in the linear index row*K + col (sorted row-major, no
 *     duplicates).  0 <= row < M, 0 <= col < K.
 *   - dtype: values and activations share one element type, SNACK_F32
 *     (float) or SNACK_BF16 (raw bfloat16 bits, uint16).  Products
 *     accumulate in fp32 and round once (to nearest even) to the output type.
 *   - layout: activations of F features and batch B are either batch-major
 *     (B x F, element [b*F + f]) or node-major (F x B, element [f*B + b]).
 *     Outputs use the same layout as the inputs.
 *   - memory: every array argument is caller-owned device memory unless
 *     stated otherwise.  The library allocates no memory (device or pinned
 *     host) and keeps no global state, with two exceptions: the code object
 *     of a generated fixed-pattern kernel (snack_fixed_build), owned by its
 *     handle, and the per-GPU workspace array of snack_prune_regrow_static.
 *     Plans are caller-owned host structs.
 *   - streams: `stream` is a hipStream_t (NULL = the null stream).  All
 *     calls are stream-ordered and asynchronous, except snack_coo_prepare
 *     and snack_prune_regrow(_prepared), which read a few words back and
 *     wait for the stream before returning.  With a plan whose host_words
 *     point to caller-owned pinned host memory, the kernels store those
 *     words straight into it and the host spins on a completion word that a
 *     last, one-thread kernel stores (falling back to hipStreamSynchronize
 *     after 20 ms); the calling thread is busy while it waits.  Otherwise the
 *     words are copied back and the stream synchronised.
 *   - errors: a negative snack_status.  Argument errors are detected on the
 *     host before anything is launched and leave every output untouched.
 *     Nothing aborts or prints.
 *   - concurrency: calls that share a plan's arena, or a workspace, must
 *     not overlap (they write the same scratch).
 *   - debug build: libsnack_debug.so exports this same ABI; before any
 *     product kernel its product entry points check, on the device and on
 *     the call's stream, every plan array and COO index the kernels take
 *     indices from (offsets from 0 to nnz and non-decreasing, indices and
 *     perm in range, tiles and cut flags well formed), reading each array
 *     only within the size the plan gives it, and return
 *     SNACK_E_PLAN_CORRUPT without launching anything else on a violation.
 *     Each product call then also synchronises its stream once.
 */
#ifndef SNACK_H_
#define SNACK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define SNACK_API __attribute__((visibility("default")))
#else
#define SNACK_API
#endif

typedef int32_t snack_status;

#define SNACK_OK 0
#define SNACK_E_NULL (-1)          /* a required pointer is NULL */
#define SNACK_E_SHAPE (-2)         /* M, K, B, nnz or tile size out of range */
#define SNACK_E_DTYPE (-3)         /* unknown dtype */
#define SNACK_E_LAYOUT (-4)        /* unknown layout */
#define SNACK_E_COO_RANGE (-5)     /* a COO index lies outside [0,M) x [0,K) */
#define SNACK_E_COO_ORDER (-6)     /* COO not strictly increasing (unsorted or duplicate) */
#define SNACK_E_NAN (-7)           /* a NaN value where magnitudes are compared */
#define SNACK_E_COUNT (-8)         /* n_drop > nnz or n_drop > M*K - nnz */
#define SNACK_E_WORKSPACE (-9)     /* arena / workspace too small */
#define SNACK_E_OVERFLOW (-10)     /* a size exceeds the int32 index range */
#define SNACK_E_HIP (-11)          /* a HIP launch or runtime call failed */
#define SNACK_E_NOT_PREPARED (-12) /* the plan has not been prepared */
#define SNACK_E_PLAN_CORRUPT (-13) /* debug build only: a plan array or COO index failed
                                      the device check run before a product */

/* Element type and activation layout are plain int32 arguments (any value
 * may be passed and is checked: SNACK_E_DTYPE / SNACK_E_LAYOUT). */
typedef int32_t snack_dtype;
enum { SNACK_F32 = 0, SNACK_BF16 = 1 };
typedef int32_t snack_layout;
enum { SNACK_BATCH_MAJOR = 0, SNACK_NODE_MAJOR = 1 };

/* Derived arrays of a prepared plan (see snack_plan_array). */
typedef enum {
  SNACK_ARR_ROW_PTR = 0,     /* int32 [M+1]   row-segment offsets */
  SNACK_ARR_RPART_SEG = 1,   /* int32 [P_row+1] tile start: segment (row) */
  SNACK_ARR_RPART_NZ = 2,    /* int32 [P_row+1] tile start: entry */
  SNACK_ARR_RCUT = 3,        /* int32 [P_row+1] 1 if cut p lies inside a row (long row split) */
  SNACK_ARR_COL_PTR = 4,     /* int32 [K+1]   column-segment offsets */
  SNACK_ARR_PERM = 5,        /* int32 [nnz]   row-major position of the i-th entry in (col,row) order */
  SNACK_ARR_ROW_T = 6,       /* int32 [nnz]   row[perm[i]] */
  SNACK_ARR_CPART_SEG = 7,   /* int32 [P_col+1] */
  SNACK_ARR_CPART_NZ = 8,    /* int32 [P_col+1] */
  SNACK_ARR_CCUT = 9,        /* int32 [P_col+1] 1 if cut p lies inside a column */
  SNACK_ARR_COUNT_ = 10
} snack_array;

#define SNACK_PLAN_SLOTS 16

/* Bytes of caller-owned pinned host memory a plan's host_words must hold. */
#define SNACK_HOST_WORDS_BYTES 64

/*
 * Plan: the prepared topology of one COO weight.  Filled by snack_plan_init
 * (sizes) and snack_coo_prepare (derived arrays in the caller's arena).
 * The struct is plain data; copy it freely, but the arrays live in `arena`.
 */
typedef struct snack_plan {
  int32_t M, K;              /* W is M x K (out_features x in_features) */
  int64_t nnz;
  int32_t max_batch;         /* largest B a product call on this plan may use */
  int32_t tile_row;          /* work items (entries + row ends) per row-view tile */
  int32_t tile_col;          /* work items per column-view tile */
  int32_t P_row, P_col;      /* number of tiles of each view */
  int32_t has_split_row;     /* 1 if some row spans several tiles (set by prepare) */
  int32_t has_split_col;     /* 1 if some column spans several tiles (set by prepare) */
  int32_t prepared;          /* 1 after a successful snack_coo_prepare */
  const int32_t* row;        /* device COO recorded by prepare (not owned) */
  const int32_t* col;
  void* arena;               /* device arena recorded by prepare (not owned) */
  size_t arena_bytes;        /* bytes the arena must provide (set by init) */
  size_t off[SNACK_PLAN_SLOTS]; /* byte offsets of the arrays in the arena */
  /* Optional, set by the caller after snack_plan_init: pinned, device-mapped
   * host memory of SNACK_HOST_WORDS_BYTES bytes (hipHostMalloc, or a pinned
   * torch tensor), owned by the caller and used by one call at a time.  The
   * calls that read words back (prepare, the prepared restructure) have the
   * kernels store them straight into it, with no copy; NULL: the words come
   * back by a copy and a stream sync (a few microseconds more). */
  int32_t* host_words;
  int32_t* host_words_dev;   /* device address of host_words (set by the library) */
  const int32_t* host_words_key; /* host_words that host_words_dev belongs to */
} snack_plan;

/* Library version (major*10000 + minor*100 + patch) and sizeof(snack_plan),
 * for bindings that mirror the struct. */
SNACK_API int32_t snack_version(void);
SNACK_API size_t snack_plan_sizeof(void);

/* Human-readable text of a status code (static storage). */
SNACK_API const char* snack_status_str(snack_status s);

/* snack_plan_init flags */
#define SNACK_PLAN_NODE_MAJOR_ONLY 1u /* no scratch for transposing batch-major activations */

/*
 * snack_plan_init -- host only, no device work.
 * Computes tile sizes, tile counts and the arena layout for a weight of
 * shape M x K with nnz nonzeros, for product calls with B <= max_batch.
 * tile_items = 0 picks each view's tile size automatically: the smallest
 * power of two in [128, 2048] giving at most ~2048 tiles, and for
 * max_batch > 32 also at least twice the view's mean segment length (so
 * that only segments well above the mean are cut into tile pieces, whose
 * partial sums travel through fp32 carry slots); otherwise tile_items must
 * lie in [1, 2048] and is used for both views.  Unless flags has
 * SNACK_PLAN_NODE_MAJOR_ONLY, the arena also holds 4*max_batch*(M+K) bytes
 * into which product calls copy batch-major activations (B > 1) in
 * node-major order before gathering from them.
 * Errors: SNACK_E_NULL, SNACK_E_SHAPE (M<1, K<1, nnz<0, nnz>M*K,
 * max_batch<1, bad tile), SNACK_E_OVERFLOW (nnz + max(M,K) >= 2^31),
 * SNACK_E_LAYOUT (unknown flag).
 */
SNACK_API snack_status snack_plan_init(snack_plan* plan, int32_t M, int32_t K, int64_t nnz,
                                       int32_t max_batch, int32_t tile_items, uint32_t flags);

/*
 * snack_coo_prepare -- the "device row-segment offsets and load-balanced
 * partition" of the layer, plus the column view used by the transpose
 * product.
 *
 * Builds, on the device, in `arena` (>= plan->arena_bytes bytes):
 *   row_ptr[M+1]      row_ptr[r] = number of entries in rows < r;
 *   row-view tiles    the merge path of row ends and entries cut every
 *                     tile_row items, each cut moved back to the start of its
 *                     row unless that row has >= tile_row entries (so only
 *                     long rows are ever split across tiles);
 *   cut flags         1 where a cut lies inside a (long) row;
 *   col_ptr[K+1], perm[nnz], row_t[nnz]  the column view: entries in stable
 *                     (col, row) order; perm[i] is the row-major position of
 *                     the i-th one and row_t[i] its row;
 *   column-view tiles and cut flags, as for rows.
 * The load balancing answers the imbalance the "Two Lotteries" page
 * describes (section on who does the work): every tile gets about the same
 * number of entries + segment ends, whatever the row lengths.
 * Validates the COO first: SNACK_E_COO_RANGE / SNACK_E_COO_ORDER.
 * Runs about a dozen kernels, then reads back 12 bytes (error bits and the
 * two has_split flags) and waits for `stream` (see streams above).  Records row, col and
 * arena in the plan; they must stay alive and unchanged while the plan is
 * used.  Re-run after every change of the sparsity pattern.  SNACK_E_WORKSPACE
 * if plan->host_words is set but is not pinned, device-mapped host memory.
 */
SNACK_API snack_status snack_coo_prepare(snack_plan* plan, const int32_t* row, const int32_t* col,
                               void* arena, size_t arena_bytes, void* stream);

/* Device pointer and element count of a derived array of a prepared plan
 * (NULL if not prepared or `which` is unknown). */
SNACK_API const void* snack_plan_array(const snack_plan* plan, int32_t which, int64_t* count);

/*
 * snack_spmm_fwd -- forward product of the layer, Y = X W^T:
 *     Y[b, r] = sum_{k : row[k] = r} v[k] * X[b, col[k]]
 * for b < B, r < M; rows without entries give exactly 0.  X has K features,
 * Y has M features, both in `layout`.  Y is overwritten (no bias, no beta).
 * Requires a prepared plan and 0 <= B <= plan->max_batch.  Batch-major
 * activations with B > 1 are first copied node-major into the plan's arena
 * (SNACK_E_WORKSPACE if the plan was made with SNACK_PLAN_NODE_MAJOR_ONLY).
 */
SNACK_API snack_status snack_spmm_fwd(const snack_plan* plan, const void* vals, snack_dtype dtype,
                            const void* X, snack_layout layout, int32_t B, void* Y,
                            void* stream);

/* Nonlinearity applied to each finished output of snack_spmm_fwd_act. */
typedef enum { SNACK_ACT_NONE = 0, SNACK_ACT_RELU = 1, SNACK_ACT_GELU = 2 } snack_act;

/*
 * snack_spmm_fwd_act -- snack_spmm_fwd followed by a nonlinearity:
 * Y[b, r] = act(sum_{k : row[k] = r} v[k] * X[b, col[k]]).
 * act: SNACK_ACT_NONE (identity), SNACK_ACT_RELU (max(x, 0); NaN gives 0)
 * or SNACK_ACT_GELU (exact, x * Phi(x) with the error function), the
 * nonlinearity between propagation steps of the graph-style inference the
 * SNACK abstract measures.  ReLU is applied in the product's store, to the
 * fp32 sum before its single rounding; GELU runs as one elementwise pass
 * over Y on the same stream right after the product (it reads the rounded
 * sums and rounds again).  Rows without entries give act(0) = 0.  Errors:
 * as snack_spmm_fwd, and SNACK_E_SHAPE for an unknown act.
 */
SNACK_API snack_status snack_spmm_fwd_act(const snack_plan* plan, const void* vals,
                                          snack_dtype dtype, const void* X, snack_layout layout,
                                          int32_t B, void* Y, int32_t act, void* stream);

/*
 * snack_graph_propagate -- multi-layer graph-style inference (the abstract's
 * "graph-style inference", read here as repeated propagation through one
 * sparse adjacency): H_0 = X, H_l = act(H_{l-1} W^T) for l = 1 .. layers,
 * Y = H_layers, each layer one snack_spmm_fwd_act launch on `stream`, each
 * H_l rounded to dtype.  layers > 1 needs a square plan (M == K) and tmp,
 * a device buffer of B*M elements used for alternate layers (tmp may be
 * NULL when layers == 1).  Y must not alias X or tmp.  Asynchronous.
 * Errors: as snack_spmm_fwd_act; SNACK_E_SHAPE for layers < 1, a
 * non-square plan with layers > 1, or aliasing; SNACK_E_NULL for a missing
 * tmp.
 */
SNACK_API snack_status snack_graph_propagate(const snack_plan* plan, const void* vals,
                                             snack_dtype dtype, const void* X,
                                             snack_layout layout, int32_t B, int32_t layers,
                                             int32_t act, void* Y, void* tmp, void* stream);

/*
 * snack_spmm_bwd_input -- gradient with respect to the layer input,
 * dX = dY W, kept sparse (only the nonzeros are touched):
 *     dX[b, c] = sum_{k : col[k] = c} v[k] * dY[b, row[k]]
 * computed over the column view without atomics; columns without entries
 * give exactly 0.  dY has M features, dX has K features.
 */
SNACK_API snack_status snack_spmm_bwd_input(const snack_plan* plan, const void* vals, snack_dtype dtype,
                                  const void* dY, snack_layout layout, int32_t B, void* dX,
                                  void* stream);

/*
 * Values in column order.  The input gradient walks the column view, whose
 * i-th entry is stored value perm[i]; reading vals[perm[i]] is a scattered
 * load per entry.  A caller-owned copy vals_t[i] = vals[perm[i]] (nnz
 * elements of the value dtype) lets it read the values coalesced, as the
 * forward product does.  The copy is the caller's to keep in step with the
 * values: snack_gather_vals_t writes it from vals, and the two calls that
 * write the values themselves (snack_spmm_bwd_fused's update,
 * snack_prune_regrow_prepared) can keep it as well.
 *
 * snack_gather_vals_t: vals_t[i] = vals[perm[i]] for i < nnz.  Asynchronous.
 * Errors: SNACK_E_NULL, SNACK_E_NOT_PREPARED, SNACK_E_DTYPE.
 */
SNACK_API snack_status snack_gather_vals_t(const snack_plan* plan, const void* vals,
                                           snack_dtype dtype, void* vals_t, void* stream);

/*
 * snack_spmm_bwd_input_t -- snack_spmm_bwd_input with the values given in
 * column order (vals_t as above):
 *     dX[b, c] = sum_{i : col_ptr[c] <= i < col_ptr[c+1]} vals_t[i] * dY[b, row_t[i]]
 * which equals dY W when vals_t[i] = vals[perm[i]].  Same arguments, layouts
 * and errors as snack_spmm_bwd_input.
 */
SNACK_API snack_status snack_spmm_bwd_input_t(const snack_plan* plan, const void* vals_t,
                                              snack_dtype dtype, const void* dY,
                                              snack_layout layout, int32_t B, void* dX,
                                              void* stream);

/*
 * snack_sddmm_grad_vals -- gradient with respect to the stored values
 * only, (dY^T X) sampled at the nonzeros:
 *     dV[k] = sum_{b < B} dY[b, row[k]] * X[b, col[k]]
 * dV (nnz elements of `dtype`, same order as the values) is overwritten;
 * B = 0 gives zeros.
 */
SNACK_API snack_status snack_sddmm_grad_vals(const snack_plan* plan, const void* dY, const void* X,
                                   snack_dtype dtype, snack_layout layout, int32_t B,
                                   void* dvals, void* stream);

/*
 * snack_spmm_bwd_fused -- the whole backward of the layer in one pass over
 * the column view, for batches of at most 32:
 *   dX = dY W                        (as snack_spmm_bwd_input),
 *   dvals[k] = sum_b dY[b,row_k] X[b,col_k]   (as snack_sddmm_grad_vals;
 *                                     dvals may be NULL),
 *   if lr != 0: vals[k] <- vals[k] - lr * dV_k   (plain SGD, in place; dV_k
 *                                     is the fp32 sum before rounding, the
 *                                     result is rounded to the value dtype).
 * Each entry's dY row is gathered once for both products; its X chunk is
 * read at its own column.  dX uses the values before the update.  This
 * follows the SNACK abstract's wish to keep backpropagation in the sparse
 * paradigm; fusing it with the optimiser is this library's.
 * X, dY: activations of the forward (B x K / B x M, or node-major); dX as
 * for snack_spmm_bwd_input.  vals_t (nullable): the values in column order
 * (vals_t[i] == vals[perm[i]], see snack_gather_vals_t); when given, the
 * values are read from it coalesced, and with lr != 0 it is updated as well,
 * so it stays in step with vals.  Errors: as for the products, SNACK_E_SHAPE
 * for B > 32, SNACK_E_NAN for a NaN or infinite lr.
 */
SNACK_API snack_status snack_spmm_bwd_fused(const snack_plan* plan, void* vals, void* vals_t,
                                  snack_dtype dtype, const void* X, const void* dY,
                                  snack_layout layout, int32_t B, void* dX, void* dvals,
                                  float lr, void* stream);

/*
 * snack_spmm_bwd_fused_adam -- snack_spmm_bwd_fused with an Adam step
 * (Kingma & Ba, "Adam: A Method for Stochastic Optimization", ICLR 2015,
 * Algorithm 1) in place of SGD: with g_k the fp32 sum dV_k before rounding,
 *   m_k <- beta1 m_k + (1 - beta1) g_k,   v_k <- beta2 v_k + (1 - beta2) g_k^2,
 *   vals[k] <- RNE(vals[k] - lr (m_k c1) / (sqrt(v_k c2) + eps)),
 * c1 = 1 / (1 - beta1^step), c2 = 1 / (1 - beta2^step) (in double on the
 * host).  m_t and v_t (fp32, nnz each) hold the moments in the plan's column
 * order (entry i of the column view, as vals_t), caller-owned, zero before
 * step 1, read and written coalesced; they follow the column order of the
 * plan, so a restructure (which reorders and replaces entries) leaves them
 * to the caller to reset.  vals_t (nullable), dX, dvals (nullable): as for
 * snack_spmm_bwd_fused.  Runs in the one-wave-per-column form only: a column
 * view with columns split over tiles, or a batch that one pass does not
 * cover (odd batches above 16), gives SNACK_E_SHAPE before anything is
 * launched.  Errors: as snack_spmm_bwd_fused; SNACK_E_NULL (adam, X, or the
 * moments missing), SNACK_E_SHAPE (B < 1 or B > 32, step < 1, a beta outside
 * [0, 1), eps < 0), SNACK_E_NAN (a hyperparameter NaN or infinite).
 */
typedef struct snack_adam {
  float lr, beta1, beta2, eps;
  int32_t step;  /* t >= 1 */
} snack_adam;
SNACK_API snack_status snack_spmm_bwd_fused_adam(const snack_plan* plan, void* vals, void* vals_t,
                                                 snack_dtype dtype, const void* X, const void* dY,
                                                 snack_layout layout, int32_t B, void* dX,
                                                 void* dvals, float* m_t, float* v_t,
                                                 const snack_adam* adam, void* stream);

/*
 * snack_drop_count -- number of connections one restructuring step
 * replaces: round half up of nnz * frac_ppm / 10^6 (frac in parts per
 * million).  Returns -1 for negative arguments.
 */
SNACK_API int64_t snack_drop_count(int64_t nnz, int32_t frac_ppm);

/* Workspace bytes snack_prune_regrow needs for these sizes. */
SNACK_API snack_status snack_prune_regrow_workspace(int32_t M, int32_t K, int64_t nnz, int64_t n_drop,
                                          size_t* bytes);

/* Restructure flags (the _ex calls and snack_prune_regrow_prepared).  The
 * library runs the bitmap plan (support bitmaps over the M x K grid) when the
 * density is at most 1/4 and the bitmaps are small, else the sort plan
 * (candidates sorted by position).  SNACK_PRUNE_SORT_PLAN forces the sort
 * plan; both give identical results. */
#define SNACK_PRUNE_SORT_PLAN 1u
SNACK_API snack_status snack_prune_regrow_workspace_ex(int32_t M, int32_t K, int64_t nnz,
                                                       int64_t n_drop, uint32_t flags,
                                                       size_t* bytes);

/*
 * snack_prune_regrow -- one restructuring step of dynamic sparse training
 * (the "restructuring connections" of the SNACK abstract; the page names
 * the operation, the rule below is this library's):
 *   1. magnitude key of entry k = its value's bits with the sign cleared
 *      (-0 == +0); NaN is an error (SNACK_E_NAN);
 *   2. the n_drop entries smallest in (magnitude key, row*K+col) are dropped;
 *      survivors keep their values;
 *   3. n_drop new positions are grown: with SplitMix64 (Steele, Lea & Flood,
 *      OOPSLA 2014), x_i = output i of a generator seeded with
 *      s = output `step` of a generator seeded with `seed`;
 *      p_i = floor(x_i * (M*K) / 2^64); p_i is taken if it is not in the
 *      support before this step and was not taken before, until n_drop are
 *      taken;
 *   4. the new COO (survivors + grown, value 0) is written back in place into
 *      row/col/vals, sorted row-major; nnz is unchanged.
 * dropped_lin / grown_lin (nullable, int64 [n_drop]) receive the dropped and
 * grown linear indices in increasing order.  ws must hold
 * snack_prune_regrow_workspace bytes.  Re-run snack_coo_prepare afterwards.
 * Errors: SNACK_E_COUNT, SNACK_E_NAN (COO left unchanged), SNACK_E_WORKSPACE.
 * Synchronises `stream` (its few result words come back by a copy).
 */
SNACK_API snack_status snack_prune_regrow(int32_t* row, int32_t* col, void* vals, snack_dtype dtype,
                                int32_t M, int32_t K, int64_t nnz, int64_t n_drop,
                                uint64_t seed, uint64_t step, int64_t* dropped_lin,
                                int64_t* grown_lin, void* ws, size_t ws_bytes, void* stream);
/* The same with restructure flags (ws sized by snack_prune_regrow_workspace_ex
 * with the same flags); SNACK_E_LAYOUT for an unknown flag. */
SNACK_API snack_status snack_prune_regrow_ex(int32_t* row, int32_t* col, void* vals,
                                             snack_dtype dtype, int32_t M, int32_t K,
                                             int64_t nnz, int64_t n_drop, uint64_t seed,
                                             uint64_t step, int64_t* dropped_lin,
                                             int64_t* grown_lin, void* ws, size_t ws_bytes,
                                             uint32_t flags, void* stream);

/*
 * snack_prune_regrow_static -- snack_prune_regrow for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same step, arguments and results, with the
 * workspace taken from a device array the library holds, one per GPU,
 * SNACK_STATIC_WS_MAX bytes (32 MiB: enough for 4096 x 4096 layers at 90-99%
 * sparsity and the GPT-2-sized projections; kept until the process ends).
 * The call allocates nothing.  Layers whose snack_prune_regrow_workspace
 * exceeds the limit get SNACK_E_WORKSPACE.  Every call on one GPU shares its
 * array: calls that overlap on one GPU (several streams or host threads)
 * race and must be serialised by the caller.  Synchronises `stream`.
 */
#define SNACK_STATIC_WS_MAX (32u << 20)
SNACK_API snack_status snack_prune_regrow_static(int32_t* row, int32_t* col, void* vals,
                                                 snack_dtype dtype, int32_t M, int32_t K,
                                                 int64_t nnz, int64_t n_drop, uint64_t seed,
                                                 uint64_t step, int64_t* dropped_lin,
                                                 int64_t* grown_lin, void* stream);

/*
 * snack_prune_regrow_prepared -- snack_prune_regrow followed by
 * snack_coo_prepare of the result, in one call with one synchronisation.
 * `plan` must have been prepared (snack_coo_prepare) for a COO with the same
 * M, K and nnz; on success it describes the new COO (row/col as passed) in
 * its own arena.  When the layer has density <= 1/4 and M and K are
 * multiples of 32, the derived arrays are built straight from the support
 * bitmap of the new COO (row offsets from prefix popcounts, the column view
 * from a 32 x 32 bit-tile transpose), with no sort and no re-validation;
 * otherwise the two calls run one after the other.  Results (COO, lists,
 * derived arrays) are identical either way.  dtype, n_drop, seed, step,
 * dropped_lin, grown_lin, ws, ws_bytes, flags: as for snack_prune_regrow_ex
 * (ws sized by snack_prune_regrow_workspace_ex with the same flags).
 * vals_t (nullable, nnz elements): receives the new values in the new
 * column order (vals_t[i] = vals[perm[i]], see snack_gather_vals_t).
 * Errors: as for snack_prune_regrow_ex, plus SNACK_E_NOT_PREPARED (plan
 * never prepared).  On error the plan must be prepared again before use.
 * Synchronises `stream`.
 */
SNACK_API snack_status snack_prune_regrow_prepared(snack_plan* plan, int32_t* row, int32_t* col,
                                         void* vals, void* vals_t, snack_dtype dtype,
                                         int64_t n_drop, uint64_t seed, uint64_t step,
                                         int64_t* dropped_lin, int64_t* grown_lin, void* ws,
                                         size_t ws_bytes, uint32_t flags, void* stream);

/*
 * snack_memory_footprint -- host only: device bytes of one layer, held
 * against the same layer stored dense and as Dense+Mask (the memory
 * comparison of the SNACK abstract, which reports a sparse layer at 90%
 * sparsity using far less memory than a dense one).  For an M x K layer
 * with nnz connections of element size s (dtype), product calls up to
 * max_batch, plan flags plan_flags (as snack_plan_init, tile size automatic)
 * and restructuring steps of n_drop connections (0: no restructuring):
 *   coo            row, col (int32) and values: nnz * (8 + s)
 *   value_grad     the value gradient dV: nnz * s
 *   col_values     the values in column order that the input gradient reads
 *                  (snack_gather_vals_t): nnz * s
 *   derived        the arrays a prepared plan keeps (row offsets, column
 *                  view, tiles and cut flags of both views)
 *   plan_scratch   the rest of the plan arena (sort buffers of prepare,
 *                  carry slots, node-major copies of activations)
 *   restructure_ws snack_prune_regrow_workspace(M, K, nnz, n_drop), or 0
 *   sparse_total   the sum of the six above
 *   dense_weight, dense_grad   M * K * s each; dense_total their sum
 *   mask           a uint8 mask of the Dense+Mask layer: M * K
 *   masked_total   dense_total + mask
 *   activations    X, Y and their gradients at max_batch, the same for
 *                  all three layers: 2 * max_batch * (M + K) * s
 * No optimiser state is counted (the in-place SGD step of
 * snack_spmm_bwd_fused keeps none).  Errors: as snack_plan_init and
 * snack_prune_regrow_workspace, SNACK_E_DTYPE, SNACK_E_COUNT.
 */
typedef struct snack_footprint {
  uint64_t coo, value_grad, col_values, derived, plan_scratch, restructure_ws, sparse_total;
  uint64_t dense_weight, dense_grad, dense_total;
  uint64_t mask, masked_total;
  uint64_t activations;
} snack_footprint;

SNACK_API snack_status snack_memory_footprint(int32_t M, int32_t K, int64_t nnz,
                                              int32_t max_batch, snack_dtype dtype,
                                              int64_t n_drop, uint32_t plan_flags,
                                              snack_footprint* out);

/*
 * Fixed-pattern inference kernels (SparseRT, "Accelerating Unstructured
 * Sparsity on GPUs for Deep Learning Inference", Abstract: a code generator
 * that bakes a fixed sparse weight into the kernel, for fully connected
 * layers and 1x1 convolutions).  snack_fixed_build reads a COO weight and
 * its values from HOST memory (row, col int32 strictly increasing
 * row-major, vals float or raw bf16 bits as dtype), writes a kernel for
 * exactly that weight -- the values become immediate operands, the indices
 * become the code's structure -- compiles it with hipRTC for gfx950 and
 * loads it.  The rows are cut into bands of about 8K entries (one
 * workgroup each per 64 batch columns) and the inputs are staged in tiles
 * of 256, so any M and K work.  Limits: M, K >= 1, nnz <= 2^23, at most
 * 65535 bands (else SNACK_E_SHAPE).  Code size and build time grow linearly
 * with nnz: 13-22 bytes of code and 0.15-0.3 ms of compilation per entry (a
 * 4096 x 4096 layer at 95% sparsity takes minutes).  The handle owns the
 * loaded code object (device memory for code, the one exception to "no
 * allocation") until snack_fixed_free.  flags: SNACK_FIXED_COMPILE_ONLY
 * generates and compiles without loading (no GPU needed; the handle cannot
 * run).  Errors: SNACK_E_NULL, SNACK_E_DTYPE, SNACK_E_SHAPE,
 * SNACK_E_COO_RANGE, SNACK_E_COO_ORDER, SNACK_E_LAYOUT (unknown flag),
 * SNACK_E_HIP (compile or load failure).
 *
 * snack_fixed_fwd: Y = X W^T for `images` independent node-major blocks,
 * X[i] (K x B) at X + i*K*B and Y[i] (M x B) at Y + i*M*B, in the dtype the
 * handle was built for; fp32 accumulation, one rounding.  An NCHW 1x1
 * convolution with C_in = K, C_out = M over images of H*W pixels is this
 * call with B = H*W.  One launch, asynchronous on `stream`.  Errors:
 * SNACK_E_NULL, SNACK_E_SHAPE (negative sizes, more than 65535 images),
 * SNACK_E_NOT_PREPARED (compile-only handle).
 */
typedef struct snack_fixed snack_fixed;
#define SNACK_FIXED_COMPILE_ONLY 1u

SNACK_API snack_status snack_fixed_build(const int32_t* row, const int32_t* col, const void* vals,
                                         snack_dtype dtype, int32_t M, int32_t K, int64_t nnz,
                                         uint32_t flags, snack_fixed** out);
SNACK_API snack_status snack_fixed_fwd(const snack_fixed* f, const void* X, int32_t B,
                                       int32_t images, void* Y, void* stream);
/* Waves per workgroup, bands (workgroups per batch tile and image),
 * code-object and source sizes of a built kernel; any pointer may be NULL. */
SNACK_API snack_status snack_fixed_info(const snack_fixed* f, int32_t* waves, int32_t* bands,
                                        size_t* code_bytes, size_t* source_bytes);
/* The compiled gfx950 code object of a handle (host memory owned by it). */
SNACK_API const void* snack_fixed_code(const snack_fixed* f, size_t* bytes);
SNACK_API void snack_fixed_free(snack_fixed* f);

/*
 * snack_conv1x1 -- a 1x1 convolution with the layer's weight (C_out = M,
 * C_in = K) as products on the prepared plan: NHWC input (N*HW pixels x K
 * channels) is one batch-major snack_spmm_fwd with B = N*HW; NCHW input
 * (N images of K x HW) is one node-major snack_spmm_fwd per image with
 * B = HW.  Output in the same layout.  The plan's max_batch must cover B.
 * layout: SNACK_CONV_NHWC or SNACK_CONV_NCHW.  Errors: as snack_spmm_fwd,
 * SNACK_E_LAYOUT for an unknown layout.
 */
#define SNACK_CONV_NHWC 0
#define SNACK_CONV_NCHW 1
SNACK_API snack_status snack_conv1x1(const snack_plan* plan, const void* vals, snack_dtype dtype,
                                     const void* X, int32_t N, int32_t HW, int32_t layout, void* Y,
                                     void* stream);

/*
 * GELU with the exact error function, h = z * Phi(z), and its backward
 * dz = dh * (Phi(z) + z * phi(z)), elementwise over n fp32 values (the
 * nonlinearity between the two sparse layers of a GPT-2-shaped MLP block).
 */
SNACK_API snack_status snack_gelu_fwd(const float* z, float* h, int64_t n, void* stream);
SNACK_API snack_status snack_gelu_bwd(const float* z, const float* dh, float* dz, int64_t n,
                            void* stream);

/*
 * Dense baselines for comparison (the "Dense+Mask" and fully dense layers
 * the SNACK abstract measures against): Y = X (W .* mask)^T with a dense
 * row-major W (M x K, dtype) and an optional uint8 mask (M x K, nonzero =
 * keep; NULL = plain dense layer).  Batch-major X (B x K) and Y (B x M).
 */
SNACK_API snack_status snack_dense_fwd(const void* W, const uint8_t* mask, snack_dtype dtype, int32_t M,
                             int32_t K, const void* X, int32_t B, void* Y, void* stream);

/*
 * snack_calibrate -- the benchmark's machine floors, not part of the layer:
 *   SNACK_CALIB_EMPTY  an empty kernel of n workgroups (launch and drain);
 *   SNACK_CALIB_READ   read every 16-byte word of buf[0, bytes) once, n
 *                      workgroups (the last word is a sink that is written
 *                      only in the improbable case that the words' xor is
 *                      0x9E3779B9);
 *   SNACK_CALIB_WRITE  write zeros over buf[0, bytes), n workgroups;
 *   SNACK_CALIB_CHAIN  write a cycle of 128-byte slots into buf (a
 *                      full-period linear congruential order over the
 *                      largest power-of-two count of slots that fits);
 *   SNACK_CALIB_CHASE  one thread follows n links of that cycle, each load
 *                      depending on the last (memory latency).
 * bytes: a multiple of 16 for READ / WRITE.  Asynchronous on `stream`.
 * Errors: SNACK_E_NULL, SNACK_E_SHAPE (bad kind, size or count).
 */
#define SNACK_CALIB_EMPTY 0
#define SNACK_CALIB_READ 1
#define SNACK_CALIB_WRITE 2
#define SNACK_CALIB_CHAIN 3
#define SNACK_CALIB_CHASE 4
SNACK_API snack_status snack_calibrate(int32_t kind, void* buf, size_t bytes, int64_t n,
                                       void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SNACK_H_ */
