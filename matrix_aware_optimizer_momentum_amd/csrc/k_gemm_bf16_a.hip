// Instantiations of the batched MFMA GEMM: A operand bf16_t in HBM, MFMA input bf16_t.
#include "k_gemm.hpp"

namespace sm {

sm_status launch_gemm_bf16_a(const GemmArgs* gs, int n, int kind, hipStream_t s) {
  using namespace gemm;
  const GemmArgs& g = gs[0];
  if (g.b.dt == BF16) {
    if (g.a.layout == KC && g.b.layout == KC) return launch_t<bf16_t, bf16_t, bf16_t, KC, KC>(gs, n, kind, s);
    if (g.a.layout == KC && g.b.layout == RC) return launch_t<bf16_t, bf16_t, bf16_t, KC, RC>(gs, n, kind, s);
    if (g.a.layout == RC && g.b.layout == RC) return launch_t<bf16_t, bf16_t, bf16_t, RC, RC>(gs, n, kind, s);
  }
  if (g.b.dt == F32) {
    if (g.a.layout == KC && g.b.layout == KC) return launch_t<bf16_t, float, bf16_t, KC, KC>(gs, n, kind, s);
    if (g.a.layout == KC && g.b.layout == RC) return launch_t<bf16_t, float, bf16_t, KC, RC>(gs, n, kind, s);
    if (g.a.layout == RC && g.b.layout == RC) return launch_t<bf16_t, float, bf16_t, RC, RC>(gs, n, kind, s);
  }
  return SM_ERR_UNSUPPORTED;
}

}  // namespace sm
