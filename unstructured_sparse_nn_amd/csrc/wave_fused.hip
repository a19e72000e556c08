// wave_fused.hip -- the fused backward over the column view, one wave per
// column, for views with no split segment.
//
// For column c (a segment of the column view: entries k' in the column's
// range, their rows r = row_t[k'] and value positions p = perm[k']):
//   dX[b, c] = sum_k' v[p] dY[b, r]            (the input gradient)
//   dV[p]    = sum_b dY[b, r] X[b, c]          (the value gradient)
//   v[p]    <- RNE(v[p] - lr dV[p])            (optional SGD step, lr != 0)
// Both gradients ("Beyond Masked Sparsity: SNACK Enables Truly Sparse Neural
// Networks on GPU", Abstract: backpropagation entirely in the sparse
// paradigm) share one gather of the dY row per entry: its chunk is added,
// scaled by the value, into the column's dX sums, and dotted with the
// column's X chunk (loaded once per wave) for dV.  dV and the updated value
// are written through perm by the lane that loaded the entry.  Each value is
// read and written by that one lane only, so the in-place update races with
// nothing.  With the values also kept in column order (vals_t, VT), they are
// read from there coalesced instead of through perm, and the update writes
// both copies.
#include "common.h"
#include "internal.h"
#include "wave.h"

namespace snk {

// Optimiser step applied to each value by the fused backward.
enum { OPT_SGD = 0, OPT_ADAM = 1 };
// Adam (Kingma & Ba, ICLR 2015, Algorithm 1) with the bias corrections
// c1 = 1 / (1 - beta1^t), c2 = 1 / (1 - beta2^t) taken on the host.
struct adam_hp {
  float lr, b1, b2, eps, c1, c2;
};

template <typename T, int CH, int LPE, int NR, bool VT, int OPT>
__device__ __forceinline__ void fused_rounds(const T* __restrict__ gb, int32_t B,
                                             const vec<T, CH>& xs, const int32_t* ci,
                                             const float* cv, const int32_t* pk, int32_t rb,
                                             int32_t e, int lane, int slot, float (&acc)[CH],
                                             T* __restrict__ dV, T* vals_upd, T* vals_t,
                                             float lr, const float* mq, const float* vq,
                                             float* __restrict__ m_t, float* __restrict__ v_t,
                                             const adam_hp& hp) {
  constexpr int NQ = (NR + LPE - 1) / LPE;
  vec<T, CH> gv[NR];
  float vj[NR];
  gather_rounds<T, CH, LPE, NR>(gb, B, ci, cv, rb, e, slot, gv, vj);
  accumulate_rounds<T, CH, NR>(gv, vj, acc);
  float d[NQ];
  round_dots<T, CH, LPE, NR>(gv, xs, lane, d);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int32_t k = rb + q * SNK_WAVE + lane;
    if (k < e) {
      if (dV) dV[pk[q]] = elem<T>::from_f(d[q]);
      if constexpr (OPT == OPT_ADAM) {
        const float g = d[q];
        const float m = hp.b1 * mq[q] + (1.f - hp.b1) * g;
        const float v = hp.b2 * vq[q] + (1.f - hp.b2) * g * g;
        m_t[k] = m;
        v_t[k] = v;
        const T u = elem<T>::from_f(cv[q] - hp.lr * (m * hp.c1) / (sqrtf(v * hp.c2) + hp.eps));
        vals_upd[pk[q]] = u;
        if constexpr (VT) vals_t[k] = u;
      } else if (lr != 0.f) {
        const T u = elem<T>::from_f(cv[q] - lr * d[q]);
        vals_upd[pk[q]] = u;
        if constexpr (VT) vals_t[k] = u;
      }
    }
  }
}

// The fused kernel's entry loads with the values in column order: index,
// value position and value, all at the entry's own (coalesced) position.
template <typename T>
__device__ __forceinline__ void load_entries_vt(const int32_t* __restrict__ idx,
                                                const int32_t* __restrict__ perm,
                                                const T* vals_t, int32_t base, int32_t e,
                                                int lane, int32_t (&ci)[WV_U],
                                                float (&cv)[WV_U], int32_t (&pk)[WV_U]) {
  int32_t kc[WV_U];
  T raw[WV_U];
#pragma unroll
  for (int q = 0; q < WV_U; ++q) kc[q] = min(base + q * SNK_WAVE + lane, e - 1);
#pragma unroll
  for (int q = 0; q < WV_U; ++q) ci[q] = idx[kc[q]];
#pragma unroll
  for (int q = 0; q < WV_U; ++q) pk[q] = perm[kc[q]];
#pragma unroll
  for (int q = 0; q < WV_U; ++q) raw[q] = vals_t[kc[q]];
#pragma unroll
  for (int q = 0; q < WV_U; ++q)
    cv[q] = (base + q * SNK_WAVE + lane < e) ? elem<T>::to_f(raw[q]) : 0.f;
}

// One pass covers the batch: B <= LPE * CH.  Adam's moments m_t, v_t are
// fp32 arrays in column order, loaded with the entries and written back
// coalesced.
template <typename T, int CH, int LPE, bool NODE_OUT, bool VT, int OPT>
__global__ __launch_bounds__(WV_THREADS) void k_wave_bwd_fused(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ perm, T* vals, T* vals_t, const T* __restrict__ dYt,
    const T* __restrict__ Xt, T* __restrict__ dX, T* __restrict__ dV, float lr, int32_t S,
    int32_t B, int32_t xcd_blocks, float* __restrict__ m_t, float* __restrict__ v_t,
    adam_hp hp) {
  constexpr int EPI = SNK_WAVE / LPE;
  constexpr int RG = wave_rg<LPE>();
  static_assert(CH <= EPI, "reduce-scatter needs CH <= 64 / LPE");
  const int32_t s = wave_segment(xcd_blocks);
  if (s >= S) return;
  const int lane = lane_id();
  const int slot = lane / LPE;
  const int sub = lane % LPE;
  const int32_t b0 = sub * CH;
  const bool bvalid = b0 < B;
  const T* __restrict__ gb = dYt + (bvalid ? b0 : 0);
  vec<T, CH> xs = *reinterpret_cast<const vec<T, CH>*>(Xt + (int64_t)s * B + (bvalid ? b0 : 0));
  zero_unless<T, CH>(xs, bvalid);
  const int32_t a = ptr[s], e = ptr[s + 1];

  float acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) acc[c] = 0.f;

  for (int32_t base = a; base < e; base += WV_U * SNK_WAVE) {
    int32_t ci[WV_U], pk[WV_U];
    float cv[WV_U];
    if constexpr (VT) load_entries_vt<T>(idx, perm, vals_t, base, e, lane, ci, cv, pk);
    else load_entries<T, true, true>(idx, perm, vals, base, e, lane, ci, cv, pk);
    float mq[WV_U], vq[WV_U];
    if constexpr (OPT == OPT_ADAM) {
#pragma unroll
      for (int q = 0; q < WV_U; ++q) {
        const int32_t kc = min(base + q * SNK_WAVE + lane, e - 1);
        mq[q] = m_t[kc];
        vq[q] = v_t[kc];
      }
    }
#pragma unroll
    for (int g = 0; g < WV_U * LPE / RG; ++g) {
      const int q0 = g * RG / LPE;
      const int32_t rb = base + g * RG * EPI;
      if (rb >= e) break;
      const int nr = (e - rb + EPI - 1) / EPI;
      with_count<RG>(nr, [&](auto n) {
        fused_rounds<T, CH, LPE, decltype(n)::value, VT, OPT>(
            gb, B, xs, ci + q0, cv + q0, pk + q0, rb, e, lane, slot, acc, dV, vals, vals_t, lr,
            mq + q0, vq + q0, m_t, v_t, hp);
      });
    }
  }

  const int c = reduce_scatter<CH, LPE>(acc, lane);
  constexpr int LOW = EPI / CH;
  if ((slot % LOW) == 0 && bvalid) {
    const int32_t b = b0 + c;
    if constexpr (NODE_OUT) dX[(int64_t)s * B + b] = elem<T>::from_f(acc[0]);
    else dX[(int64_t)b * S + s] = elem<T>::from_f(acc[0]);
  }
}

template <typename T, int CH, int LPE, bool NODE_OUT, int OPT>
static void wave_fused_o(const seg_view& v, void* vals, void* vals_t, const void* dYt,
                         const void* Xt, int32_t B, void* dX, void* dV, float lr, dim3 grid,
                         int32_t xb, float* m_t, float* v_t, const adam_hp& hp, hipStream_t s) {
  if (vals_t)
    hipLaunchKernelGGL((k_wave_bwd_fused<T, CH, LPE, NODE_OUT, true, OPT>), grid,
                       dim3(WV_THREADS), 0, s, v.ptr, v.idx, v.perm, (T*)vals, (T*)vals_t,
                       (const T*)dYt, (const T*)Xt, (T*)dX, (T*)dV, lr, v.S, B, xb, m_t, v_t, hp);
  else
    hipLaunchKernelGGL((k_wave_bwd_fused<T, CH, LPE, NODE_OUT, false, OPT>), grid,
                       dim3(WV_THREADS), 0, s, v.ptr, v.idx, v.perm, (T*)vals, (T*)nullptr,
                       (const T*)dYt, (const T*)Xt, (T*)dX, (T*)dV, lr, v.S, B, xb, m_t, v_t, hp);
}

template <typename T, int CH, int LPE>
static void wave_fused_l(const seg_view& v, void* vals, void* vals_t, const void* dYt,
                         const void* Xt, int32_t B, void* dX, void* dV, float lr, bool node_out,
                         float* m_t, float* v_t, const adam_hp* hp, hipStream_t s) {
  const int32_t nblk = (int32_t)cdiv(v.S, WV_THREADS / SNK_WAVE);
  // die-contiguous column ranges: a line of the row-ordered arrays accessed
  // through perm (values read, dV and updated values written) is touched by
  // few dies instead of all eight
  const int32_t xb = nblk >= 8 * NUM_XCD ? (int32_t)cdiv(nblk, NUM_XCD) : 0;
  dim3 grid((unsigned)(xb ? xb * NUM_XCD : nblk));
  const adam_hp none{};
  if (hp) {
    if (node_out)
      wave_fused_o<T, CH, LPE, true, OPT_ADAM>(v, vals, vals_t, dYt, Xt, B, dX, dV, 0.f, grid,
                                               xb, m_t, v_t, *hp, s);
    else
      wave_fused_o<T, CH, LPE, false, OPT_ADAM>(v, vals, vals_t, dYt, Xt, B, dX, dV, 0.f, grid,
                                                xb, m_t, v_t, *hp, s);
  } else if (node_out) {
    wave_fused_o<T, CH, LPE, true, OPT_SGD>(v, vals, vals_t, dYt, Xt, B, dX, dV, lr, grid, xb,
                                            nullptr, nullptr, none, s);
  } else {
    wave_fused_o<T, CH, LPE, false, OPT_SGD>(v, vals, vals_t, dYt, Xt, B, dX, dV, lr, grid, xb,
                                             nullptr, nullptr, none, s);
  }
}

template <typename T, int CH>
static bool wave_fused_c(const seg_view& v, void* vals, void* vals_t, const void* dYt,
                         const void* Xt, int32_t B, void* dX, void* dV, float lr, bool node_out,
                         int lpe, float* m_t, float* v_t, const adam_hp* hp, hipStream_t s) {
#define SNK_WF(L) wave_fused_l<T, CH, L>(v, vals, vals_t, dYt, Xt, B, dX, dV, lr, node_out, m_t, v_t, hp, s)
  switch (lpe) {
    case 1: SNK_WF(1); return true;
    case 2: SNK_WF(2); return true;
    case 4: SNK_WF(4); return true;
    case 8: SNK_WF(8); return true;
    case 16:
      if constexpr (CH <= 4) {
        SNK_WF(16);
        return true;
      }
      return false;
    default: return false;
  }
#undef SNK_WF
}

bool launch_wave_bwd_fused(const seg_view& v, void* vals, void* vals_t, snack_dtype dt,
                           const void* dYt, const void* Xt, int32_t B, void* dX, void* dV,
                           float lr, bool node_out, hipStream_t s, float* m_t, float* v_t,
                           const float* adam) {
  const wave_shape w = wave_pick(dt, B);
  if ((int64_t)w.ch * w.lpe < B) return false;  // one pass must cover the batch
  adam_hp hp{};
  if (adam) hp = adam_hp{adam[0], adam[1], adam[2], adam[3], adam[4], adam[5]};
  const adam_hp* hpp = adam ? &hp : nullptr;
#define SNK_WFC(TT, C) \
  return wave_fused_c<TT, C>(v, vals, vals_t, dYt, Xt, B, dX, dV, lr, node_out, w.lpe, m_t, v_t, hpp, s)
  if (dt == SNACK_F32) {
    switch (w.ch) {
      case 1: SNK_WFC(float, 1);
      case 2: SNK_WFC(float, 2);
      default: SNK_WFC(float, 4);
    }
  }
  switch (w.ch) {
    case 1: SNK_WFC(bf16, 1);
    case 2: SNK_WFC(bf16, 2);
    case 4: SNK_WFC(bf16, 4);
    default: SNK_WFC(bf16, 8);
  }
#undef SNK_WFC
}

}  // namespace snk
