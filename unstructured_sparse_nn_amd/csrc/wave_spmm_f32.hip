// wave_spmm_f32.hip -- fp32 instantiations of the wave-per-segment products.
#include "wave_kernels.h"

namespace snk {

void wave_spmm_f32(const seg_view& v, const void* vals, const void* Xt, int32_t B, void* Y,
                   bool node_out, int32_t act, float* carry, hipStream_t s) {
  wave_spmm_d<float>(v, vals, Xt, B, Y, node_out, act, wave_pick(SNACK_F32, B), carry, s);
}

}  // namespace snk
