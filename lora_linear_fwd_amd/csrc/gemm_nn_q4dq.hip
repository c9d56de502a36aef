// LoRA GEMM instantiations for the B_NN_Q4DQ operand form (4-bit weight with
// double-quantised block constants).
#include "gemm_launch.hpp"

namespace lora {
hipError_t launch_gemm_nn_q4dq(int epi, const GemmArgs &a, hipStream_t st) {
  if (epi == EPI_STORE) return launch_gemm_t<B_NN_Q4DQ, EPI_STORE>(a, st);
  if (epi == EPI_SWIGLU_BWD) return launch_gemm_t<B_NN_Q4DQ, EPI_SWIGLU_BWD>(a, st);
  return hipErrorInvalidValue;
}
}  // namespace lora
