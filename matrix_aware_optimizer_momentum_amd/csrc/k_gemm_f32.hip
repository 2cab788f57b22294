// Instantiations of the batched MFMA GEMM: A operand float in HBM, MFMA input float.
#include "k_gemm.hpp"

namespace sm {

sm_status launch_gemm_f32(const GemmArgs* gs, int n, int kind, hipStream_t s) {
  using namespace gemm;
  const GemmArgs& g = gs[0];
  if (g.b.dt == F32) {
    if (g.a.layout == KC && g.b.layout == KC) return launch_t<float, float, float, KC, KC>(gs, n, kind, s);
    if (g.a.layout == KC && g.b.layout == RC) return launch_t<float, float, float, KC, RC>(gs, n, kind, s);
    if (g.a.layout == RC && g.b.layout == RC) return launch_t<float, float, float, RC, RC>(gs, n, kind, s);
  }
  return SM_ERR_UNSUPPORTED;
}

}  // namespace sm
