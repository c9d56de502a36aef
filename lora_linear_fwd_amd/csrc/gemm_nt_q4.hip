// LoRA GEMM instantiations for the B_NT_Q4 operand form.
#include "gemm_launch.hpp"

namespace lora {
hipError_t launch_gemm_nt_q4(int epi, const GemmArgs &a, hipStream_t st) {
  if (epi == EPI_STORE) return launch_gemm_t<B_NT_Q4, EPI_STORE>(a, st);
  if (epi == EPI_SWIGLU_FWD) return launch_gemm_t<B_NT_Q4, EPI_SWIGLU_FWD>(a, st);
  return hipErrorInvalidValue;
}
}  // namespace lora
