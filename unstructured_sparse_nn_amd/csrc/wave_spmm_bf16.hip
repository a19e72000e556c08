// wave_spmm_bf16.hip -- bf16 instantiations of the wave-per-segment products.
#include "wave_kernels.h"

namespace snk {

void wave_spmm_bf16(const seg_view& v, const void* vals, const void* Xt, int32_t B, void* Y,
                    bool node_out, int32_t act, float* carry, hipStream_t s) {
  wave_spmm_d<bf16>(v, vals, Xt, B, Y, node_out, act, wave_pick(SNACK_BF16, B), carry, s);
}

}  // namespace snk
