// LoRA GEMM instantiations for the B_NT operand form.
#include "gemm_launch.hpp"

namespace lora {
template <int PF>
static hipError_t launch_nt_pf(int epi, const GemmArgs &a, hipStream_t st) {
  if (epi == EPI_STORE) return launch_gemm_t<B_NT, EPI_STORE, PF>(a, st);
  if (epi == EPI_SWIGLU_FWD) return launch_gemm_t<B_NT, EPI_SWIGLU_FWD, PF>(a, st);
  if (epi == EPI_SWIGLU_BWD) return launch_gemm_t<B_NT, EPI_SWIGLU_BWD, PF>(a, st);
  return hipErrorInvalidValue;
}
hipError_t launch_gemm_nt(int epi, const GemmArgs &a, hipStream_t st) {
  if constexpr (kNtPrefetch) {
    if (a.K >= kPrefetchMinK) return launch_nt_pf<1>(epi, a, st);
  }
  return launch_nt_pf<0>(epi, a, st);
}
}  // namespace lora
