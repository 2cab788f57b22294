// Dispatch of the batched MFMA GEMM over operand types and layouts.
#include "k_gemm.hpp"

namespace sm {

sm_status launch_gemm_bf16_a(const GemmArgs& g, int kind, hipStream_t s);
sm_status launch_gemm_bf16_b(const GemmArgs& g, int kind, hipStream_t s);
sm_status launch_gemm_f32(const GemmArgs& g, int kind, hipStream_t s);

int gemm_tiles(int mfma_dt, int M, int N) {
  (void)mfma_dt;
  return ((M + gemm::BM - 1) / gemm::BM) * ((N + gemm::BN - 1) / gemm::BN);
}

sm_status launch_gemm(const GemmArgs& g, int mfma_dt, int kind, hipStream_t s) {
  if (g.batch <= 0 || g.M <= 0 || g.N <= 0 || g.K <= 0) return SM_OK;
  if (g.batch > 65535) return SM_ERR_SHAPE;
  if (mfma_dt == BF16) {
    if (g.a.dt == BF16) return launch_gemm_bf16_a(g, kind, s);
    return launch_gemm_bf16_b(g, kind, s);
  }
  if (g.a.dt != F32 || g.b.dt != F32) return SM_ERR_UNSUPPORTED;
  return launch_gemm_f32(g, kind, s);
}

}  // namespace sm
