// wave_sddmm_f32.hip -- fp32 instantiations of the wave-per-segment value gradient.
#include "wave_kernels.h"

namespace snk {

bool wave_sddmm_f32(const seg_view& v, const void* dYt, const void* Xt, int32_t B, void* dV,
                    hipStream_t s) {
  const wave_shape w = wave_pick(SNACK_F32, B);
  switch (w.ch) {
    case 1: return wave_sddmm_c<float, 1>(v, dYt, Xt, B, dV, w.lpe, s);
    case 2: return wave_sddmm_c<float, 2>(v, dYt, Xt, B, dV, w.lpe, s);
    default: return wave_sddmm_c<float, 4>(v, dYt, Xt, B, dV, w.lpe, s);
  }
}

}  // namespace snk
