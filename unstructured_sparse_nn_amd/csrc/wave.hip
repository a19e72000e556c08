// wave.hip -- wave-per-segment products for views whose segments all fit in
// one tile (no segment is split), the common case of uniformly sparse layers.
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
//   * its indices and values are read 64 entries per load, coalesced, up to
//     four loads in flight;
//   * lanes are split into EPI = 64 / LPE entry slots of LPE lanes; each lane
//     owns CH consecutive batch columns, so one round gathers the node-major
//     activation rows of EPI entries (LPE * CH * elem bytes per entry);
//   * the index and value of each slot's entry come from the loading lane by
//     a cross-lane permute;
//   * at the end, the EPI partial sums of each batch column are added by a
//     butterfly reduce-scatter: each exchange step halves the values a lane
//     holds, CH - 1 + log2(EPI / CH) shuffles in all instead of CH log2(EPI).
// A fixed reduction tree: results are bitwise reproducible.  Measured at
// 4096^2, 95%, batch 32 bf16, the merge-path kernel spent about 4.7 wave
// instructions per stored entry on that bookkeeping; this one spends
// about 1.5.
#include <cstdlib>
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
// are in flight together.  Values past the end are 0.
template <typename T, bool PERM, bool VALS>
__device__ __forceinline__ void load_entries(const int32_t* __restrict__ idx,
                                             const int32_t* __restrict__ perm,
                                             const T* __restrict__ vals, int32_t base, int32_t e,
                                             int lane, int32_t (&ci)[WV_U], float (&cv)[WV_U]) {
  int32_t kc[WV_U];
#pragma unroll
  for (int q = 0; q < WV_U; ++q) kc[q] = min(base + q * SNK_WAVE + lane, e - 1);
#pragma unroll
  for (int q = 0; q < WV_U; ++q) ci[q] = idx[kc[q]];
  if constexpr (VALS) {
    T raw[WV_U];
    if constexpr (PERM) {
      int32_t pk[WV_U];
#pragma unroll
      for (int q = 0; q < WV_U; ++q) pk[q] = perm[kc[q]];
#pragma unroll
      for (int q = 0; q < WV_U; ++q) raw[q] = vals[pk[q]];
    } else {
#pragma unroll
      for (int q = 0; q < WV_U; ++q) raw[q] = vals[kc[q]];
    }
#pragma unroll
    for (int q = 0; q < WV_U; ++q)
      cv[q] = (base + q * SNK_WAVE + lane < e) ? elem<T>::to_f(raw[q]) : 0.f;
  }
}

// Gather rounds issued together before any is consumed: at most 16 (one
// gathered chunk each per lane), never more than one loaded batch holds.
template <int LPE>
constexpr int wave_rg() {
  return 4 * LPE < 16 ? 4 * LPE : 16;
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
// takes chunk i / LPE, lanes (i % LPE) * EPI + slot).  Every gather first,
// then the FMAs; only the last round can hold entries past the end.
template <typename T, int CH, int LPE, int NR>
__device__ __forceinline__ void spmm_rounds(const T* __restrict__ xb, int32_t B,
                                            const int32_t* ci, const float* cv, int32_t rb,
                                            int32_t e, int slot, float (&acc)[CH]) {
  constexpr int EPI = SNK_WAVE / LPE;
  vec<T, CH> xv[NR];
  float vj[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int q = i / LPE, src = (i % LPE) * EPI + slot;
    const int32_t cj = LPE == 1 ? ci[q] : __shfl(ci[q], src, SNK_WAVE);
    vj[i] = LPE == 1 ? cv[q] : __shfl(cv[q], src, SNK_WAVE);
    xv[i] = *reinterpret_cast<const vec<T, CH>*>(xb + (int64_t)cj * B);
  }
  zero_unless<T, CH>(xv[NR - 1], rb + (NR - 1) * EPI + slot < e);
  if constexpr (sizeof(T) == 2 && CH >= 2) {
    // bf16: rounds i and i+1 together, acc[c] += v_i x_i[c] + v_i+1 x_i+1[c]
    // in one v_dot2_f32_bf16 per column; the pairs (x_i[c], x_i+1[c]) come
    // from one byte permute of the two gathered words (a bf16 value v is the
    // high half of its fp32 widening, so (v_i, v_i+1) is a permute too)
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

template <typename T, int CH, int LPE, bool PERM, bool NODE_OUT, int ACT>
__global__ __launch_bounds__(WV_THREADS) void k_wave_spmm(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm, const T* __restrict__ vals, const T* __restrict__ Xt,
    T* __restrict__ Y, int32_t S, int32_t B, int32_t xcd_blocks) {
  constexpr int EPI = SNK_WAVE / LPE;  // entries per gather round
  constexpr int RG = wave_rg<LPE>();   // rounds per group (a whole number of chunks)
  static_assert(CH <= EPI, "reduce-scatter needs CH <= 64 / LPE");
  const int32_t s = wave_segment(xcd_blocks);
  if (s >= S) return;
  const int lane = lane_id();
  const int slot = lane / LPE;
  const int sub = lane % LPE;
  const int32_t b0 = (int32_t)blockIdx.y * (LPE * CH) + sub * CH;
  const bool bvalid = b0 < B;
  const T* __restrict__ xb = Xt + (bvalid ? b0 : 0);  // lanes past the batch read column 0
  const int32_t a = ptr[s], e = ptr[s + 1];

  float acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) acc[c] = 0.f;

  for (int32_t base = a; base < e; base += WV_U * SNK_WAVE) {
    int32_t ci[WV_U];
    float cv[WV_U];
    load_entries<T, PERM, true>(idx, perm, vals, base, e, lane, ci, cv);
#pragma unroll
    for (int g = 0; g < WV_U * LPE / RG; ++g) {
      const int q0 = g * RG / LPE;
      const int32_t rb = base + g * RG * EPI;  // first entry of the group (wave-uniform)
      if (rb >= e) break;
      const int nr = (e - rb + EPI - 1) / EPI;
      with_count<RG>(nr, [&](auto n) {
        spmm_rounds<T, CH, LPE, decltype(n)::value>(xb, B, ci + q0, cv + q0, rb, e, slot, acc);
      });
    }
  }

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

// The value gradient of NR rounds: every gather first, then the dots and the
// LPE-lane sums, then per chunk of 64 entries one permute to lane = entry
// and one coalesced store.
template <typename T, int CH, int LPE, int NR>
__device__ __forceinline__ void sddmm_rounds(const T* __restrict__ xb, int32_t B,
                                             const vec<T, CH>& g, const int32_t* ci,
                                             int32_t rb, int32_t e, int lane, int slot,
                                             T* __restrict__ dV) {
  constexpr int EPI = SNK_WAVE / LPE;
  constexpr int NQ = (NR + LPE - 1) / LPE;  // chunks touched
  vec<T, CH> xv[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int q = i / LPE, src = (i % LPE) * EPI + slot;
    const int32_t cj = LPE == 1 ? ci[q] : __shfl(ci[q], src, SNK_WAVE);
    xv[i] = *reinterpret_cast<const vec<T, CH>*>(xb + (int64_t)cj * B);
  }
  float res[NQ * LPE];
#pragma unroll
  for (int i = 0; i < NQ * LPE; ++i) {
    float d = 0.f;
    if (i < NR) {
      d = dot_acc<T, CH>(g, xv[i], 0.f);
#pragma unroll
      for (int off = 1; off < LPE; off <<= 1) d += __shfl_xor(d, off, SNK_WAVE);
    }
    res[i] = d;
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    // entry q*64 + lane was dotted in round lane / EPI by slot lane % EPI
    float out = res[q * LPE];
    if constexpr (LPE > 1) {
      const int from = (lane % EPI) * LPE;
#pragma unroll
      for (int j = 0; j < LPE; ++j) {
        const float v = __shfl(res[q * LPE + j], from, SNK_WAVE);
        if (lane / EPI == j) out = v;
      }
    }
    const int32_t k = rb + q * SNK_WAVE + lane;
    if (k < e) dV[k] = elem<T>::from_f(out);
  }
}

// dV[k] for the entries of one row per wave: the row's dY chunk is loaded
// once, each round gathers EPI entries' X chunks and dots them with it, the
// LPE lanes of a slot add their partial dots, and every 64 entries the
// results are permuted to lane = entry and stored coalesced.  B <= LPE * CH.
template <typename T, int CH, int LPE>
__global__ __launch_bounds__(WV_THREADS) void k_wave_sddmm(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const T* __restrict__ dYt, const T* __restrict__ Xt, T* __restrict__ dV, int32_t S,
    int32_t B) {
  constexpr int EPI = SNK_WAVE / LPE;
  constexpr int RG = wave_rg<LPE>();
  const int32_t s = wave_segment(0);
  if (s >= S) return;
  const int lane = lane_id();
  const int slot = lane / LPE;
  const int sub = lane % LPE;
  const int32_t b0 = sub * CH;
  const bool bvalid = b0 < B;
  const int32_t a = ptr[s], e = ptr[s + 1];
  if (a == e) return;
  const T* __restrict__ xb = Xt + (bvalid ? b0 : 0);

  vec<T, CH> g = *reinterpret_cast<const vec<T, CH>*>(dYt + (int64_t)s * B + (bvalid ? b0 : 0));
  zero_unless<T, CH>(g, bvalid);

  for (int32_t base = a; base < e; base += WV_U * SNK_WAVE) {
    int32_t ci[WV_U];
    float unused[WV_U];
    load_entries<T, false, false>(idx, nullptr, (const T*)nullptr, base, e, lane, ci, unused);
#pragma unroll
    for (int gi = 0; gi < WV_U * LPE / RG; ++gi) {
      const int q0 = gi * RG / LPE;
      const int32_t rb = base + gi * RG * EPI;
      if (rb >= e) break;
      const int nr = (e - rb + EPI - 1) / EPI;
      with_count<RG>(nr, [&](auto n) {
        sddmm_rounds<T, CH, LPE, decltype(n)::value>(xb, B, g, ci + q0, rb, e, lane, slot, dV);
      });
    }
  }
}

// ---------------------------------------------------------------- host side
struct wave_shape {
  int ch;   // batch columns per lane
  int lpe;  // lanes per entry
};

// Widest lane chunk dividing B (16-byte gathers at most), then the fewest
// lanes per entry that cover the batch, capped at 64 batch columns per pass.
static wave_shape wave_pick(snack_dtype dt, int32_t B) {
  const int chmax = dt == SNACK_BF16 ? 8 : 4;
  int ch = 1;
  while (ch < chmax && B % (ch * 2) == 0) ch *= 2;
  int lpe = 1;
  while (lpe * ch < B && lpe * ch < 64) lpe *= 2;
  return {ch, lpe};
}

// Up to 16 lanes per entry (odd batches above 16 columns take the
// merge-path kernels, whose lane groups suit them better).
bool wave_eligible(const seg_view& v, snack_dtype dt, int32_t B) {
  static const bool off = getenv("SNACK_NO_WAVE") != nullptr;
  return !off && !v.has_split && wave_pick(dt, B).lpe <= 16;
}

template <typename T, int CH, int LPE, bool PERM, bool NODE_OUT, int ACT>
static void wave_spmm_t(const seg_view& v, const void* vals, const void* Xt, int32_t B, void* Y,
                        hipStream_t s) {
  const int32_t nblk = (int32_t)cdiv(v.S, WV_THREADS / SNK_WAVE);
  const int32_t xb = (PERM && nblk >= 8 * NUM_XCD) ? (int32_t)cdiv(nblk, NUM_XCD) : 0;
  dim3 grid((unsigned)(xb ? xb * NUM_XCD : nblk), (unsigned)cdiv(B, LPE * CH));
  hipLaunchKernelGGL((k_wave_spmm<T, CH, LPE, PERM, NODE_OUT, ACT>), grid, dim3(WV_THREADS), 0,
                     s, v.ptr, v.idx, v.perm, (const T*)vals, (const T*)Xt, (T*)Y, v.S, B, xb);
}

template <typename T, int CH, int LPE>
static void wave_spmm_l(const seg_view& v, const void* vals, const void* Xt, int32_t B, void* Y,
                        bool node_out, int32_t act, hipStream_t s) {
  if constexpr (CH * LPE <= 64) {
    const bool perm = v.perm != nullptr;
    if (perm) {
      if (node_out) wave_spmm_t<T, CH, LPE, true, true, ACT_NONE>(v, vals, Xt, B, Y, s);
      else wave_spmm_t<T, CH, LPE, true, false, ACT_NONE>(v, vals, Xt, B, Y, s);
    } else if (act == ACT_RELU) {
      if (node_out) wave_spmm_t<T, CH, LPE, false, true, ACT_RELU>(v, vals, Xt, B, Y, s);
      else wave_spmm_t<T, CH, LPE, false, false, ACT_RELU>(v, vals, Xt, B, Y, s);
    } else {
      if (node_out) wave_spmm_t<T, CH, LPE, false, true, ACT_NONE>(v, vals, Xt, B, Y, s);
      else wave_spmm_t<T, CH, LPE, false, false, ACT_NONE>(v, vals, Xt, B, Y, s);
    }
  }
}

template <typename T, int CH>
static void wave_spmm_c(const seg_view& v, const void* vals, const void* Xt, int32_t B, void* Y,
                        bool node_out, int32_t act, int lpe, hipStream_t s) {
  switch (lpe) {
    case 1: wave_spmm_l<T, CH, 1>(v, vals, Xt, B, Y, node_out, act, s); break;
    case 2: wave_spmm_l<T, CH, 2>(v, vals, Xt, B, Y, node_out, act, s); break;
    case 4: wave_spmm_l<T, CH, 4>(v, vals, Xt, B, Y, node_out, act, s); break;
    case 8: wave_spmm_l<T, CH, 8>(v, vals, Xt, B, Y, node_out, act, s); break;
    default: wave_spmm_l<T, CH, 16>(v, vals, Xt, B, Y, node_out, act, s); break;
  }
}

template <typename T>
static void wave_spmm_d(const seg_view& v, const void* vals, const void* Xt, int32_t B, void* Y,
                        bool node_out, int32_t act, const wave_shape& w, hipStream_t s) {
  switch (w.ch) {
    case 1: wave_spmm_c<T, 1>(v, vals, Xt, B, Y, node_out, act, w.lpe, s); break;
    case 2: wave_spmm_c<T, 2>(v, vals, Xt, B, Y, node_out, act, w.lpe, s); break;
    case 4: wave_spmm_c<T, 4>(v, vals, Xt, B, Y, node_out, act, w.lpe, s); break;
    default:
      if constexpr (sizeof(T) == 2) wave_spmm_c<T, 8>(v, vals, Xt, B, Y, node_out, act, w.lpe, s);
      break;
  }
}

void launch_wave_spmm(const seg_view& v, const void* vals, snack_dtype dt, const void* Xt,
                      int32_t B, void* Y, bool node_out, int32_t act, hipStream_t s) {
  const wave_shape w = wave_pick(dt, B);
  if (dt == SNACK_F32) wave_spmm_d<float>(v, vals, Xt, B, Y, node_out, act, w, s);
  else wave_spmm_d<bf16>(v, vals, Xt, B, Y, node_out, act, w, s);
}

template <typename T, int CH>
static bool wave_sddmm_c(const seg_view& v, const void* dYt, const void* Xt, int32_t B, void* dV,
                         int lpe, hipStream_t s) {
  dim3 grid((unsigned)cdiv(v.S, WV_THREADS / SNK_WAVE));
#define SNK_WSD(L)                                                                             \
  hipLaunchKernelGGL((k_wave_sddmm<T, CH, L>), grid, dim3(WV_THREADS), 0, s, v.ptr, v.idx,     \
                     (const T*)dYt, (const T*)Xt, (T*)dV, v.S, B)
  switch (lpe) {
    case 1: SNK_WSD(1); return true;
    case 2: SNK_WSD(2); return true;
    case 4: SNK_WSD(4); return true;
    case 8: SNK_WSD(8); return true;
    case 16: if constexpr (CH <= 4) { SNK_WSD(16); return true; } return false;
    default: return false;
  }
#undef SNK_WSD
}

bool launch_wave_sddmm(const seg_view& v, const void* dYt, const void* Xt, snack_dtype dt,
                       int32_t B, void* dV, hipStream_t s) {
  const wave_shape w = wave_pick(dt, B);
  if ((int64_t)w.ch * w.lpe < B) return false;  // one pass must cover the batch
  if (dt == SNACK_F32) {
    switch (w.ch) {
      case 1: return wave_sddmm_c<float, 1>(v, dYt, Xt, B, dV, w.lpe, s);
      case 2: return wave_sddmm_c<float, 2>(v, dYt, Xt, B, dV, w.lpe, s);
      default: return wave_sddmm_c<float, 4>(v, dYt, Xt, B, dV, w.lpe, s);
    }
  }
  switch (w.ch) {
    case 1: return wave_sddmm_c<bf16, 1>(v, dYt, Xt, B, dV, w.lpe, s);
    case 2: return wave_sddmm_c<bf16, 2>(v, dYt, Xt, B, dV, w.lpe, s);
    case 4: return wave_sddmm_c<bf16, 4>(v, dYt, Xt, B, dV, w.lpe, s);
    default: return wave_sddmm_c<bf16, 8>(v, dYt, Xt, B, dV, w.lpe, s);
  }
}

}  // namespace snk
