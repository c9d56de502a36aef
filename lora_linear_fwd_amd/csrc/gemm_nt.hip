// LoRA GEMM instantiations for the B_NT operand form.
#include "gemm_launch.hpp"

namespace lora {
hipError_t launch_gemm_nt(int epi, const GemmArgs &a, hipStream_t st) {
  const bool pf = a.K >= kPrefetchMinK;
  if (epi == EPI_STORE)
    return pf ? launch_gemm_t<B_NT, EPI_STORE, 1>(a, st) : launch_gemm_t<B_NT, EPI_STORE>(a, st);
  if (epi == EPI_SWIGLU_FWD)
    return pf ? launch_gemm_t<B_NT, EPI_SWIGLU_FWD, 1>(a, st)
              : launch_gemm_t<B_NT, EPI_SWIGLU_FWD>(a, st);
  if (epi == EPI_SWIGLU_BWD)
    return pf ? launch_gemm_t<B_NT, EPI_SWIGLU_BWD, 1>(a, st)
              : launch_gemm_t<B_NT, EPI_SWIGLU_BWD>(a, st);
  return hipErrorInvalidValue;
}
}  // namespace lora
