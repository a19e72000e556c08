// wave_sddmm_bf16.hip -- bf16 instantiations of the wave-per-segment value gradient.
#include "wave_kernels.h"

namespace snk {

bool wave_sddmm_bf16(const seg_view& v, const void* dYt, const void* Xt, int32_t B, void* dV,
                     hipStream_t s) {
  const wave_shape w = wave_pick(SNACK_BF16, B);
  switch (w.ch) {
    case 1: return wave_sddmm_c<bf16, 1>(v, dYt, Xt, B, dV, w.lpe, s);
    case 2: return wave_sddmm_c<bf16, 2>(v, dYt, Xt, B, dV, w.lpe, s);
    case 4: return wave_sddmm_c<bf16, 4>(v, dYt, Xt, B, dV, w.lpe, s);
    default: return wave_sddmm_c<bf16, 8>(v, dYt, Xt, B, dV, w.lpe, s);
  }
}

}  // namespace snk
