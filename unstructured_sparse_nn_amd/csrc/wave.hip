// wave.hip -- which products take the wave-per-segment kernels, and the
// dispatch to their per-element-type instances (the kernels themselves are
// in wave_kernels.h).
#include "common.h"
#include "internal.h"
#include "wave.h"

namespace snk {

// Per element type (wave_spmm_*.hip, wave_sddmm_*.hip), so that the many
// template instances build in parallel.
void wave_spmm_f32(const seg_view&, const void*, const void*, int32_t, void*, bool, int32_t,
                   float*, hipStream_t);
void wave_spmm_bf16(const seg_view&, const void*, const void*, int32_t, void*, bool, int32_t,
                    float*, hipStream_t);
bool wave_sddmm_f32(const seg_view&, const void*, const void*, int32_t, void*, hipStream_t);
bool wave_sddmm_bf16(const seg_view&, const void*, const void*, int32_t, void*, hipStream_t);

// ---------------------------------------------------------------- host side
// Up to 16 lanes per entry (odd batches above 16 columns take the
// merge-path kernels, whose lane groups suit them better).  Views with split
// segments qualify when the caller handles their tile pieces (split).
bool wave_eligible(const seg_view& v, snack_dtype dt, int32_t B, bool split) {
  if (wave_pick(dt, B).lpe > 16) return false;
  return !v.has_split || split;
}

void launch_wave_spmm(const seg_view& v, const void* vals, snack_dtype dt, const void* Xt,
                      int32_t B, void* Y, bool node_out, int32_t act, float* carry,
                      hipStream_t s) {
  if (dt == SNACK_F32) wave_spmm_f32(v, vals, Xt, B, Y, node_out, act, carry, s);
  else wave_spmm_bf16(v, vals, Xt, B, Y, node_out, act, carry, s);
}

bool launch_wave_sddmm(const seg_view& v, const void* dYt, const void* Xt, snack_dtype dt,
                       int32_t B, void* dV, hipStream_t s) {
  return dt == SNACK_F32 ? wave_sddmm_f32(v, dYt, Xt, B, dV, s)
                         : wave_sddmm_bf16(v, dYt, Xt, B, dV, s);
}

}  // namespace snk
