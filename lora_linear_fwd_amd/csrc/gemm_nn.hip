// LoRA GEMM instantiations for the B_NN operand form.
#include "gemm_launch.hpp"

namespace lora {
hipError_t launch_gemm_nn(int epi, const GemmArgs &a, hipStream_t st) {
  if (epi == EPI_STORE) return launch_gemm_t<B_NN, EPI_STORE>(a, st);
  if (epi == EPI_SWIGLU_BWD) return launch_gemm_t<B_NN, EPI_SWIGLU_BWD>(a, st);
  return hipErrorInvalidValue;
}
}  // namespace lora
