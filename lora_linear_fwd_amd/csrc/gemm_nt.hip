// LoRA GEMM instantiations for the B_NT operand form.
#include "gemm_launch.hpp"
#include "gemm_pp.hpp"

// 1: the eight-wave ping-pong kernel (default); 0: the four-wave kernel
#ifndef LORA_GEMM_PP
#define LORA_GEMM_PP 1
#endif

namespace lora {
#if LORA_GEMM_PP
template <int EPI>
static hipError_t launch_pp(const GemmArgs &a, hipStream_t st) {
  static std::atomic<uint64_t> done{0};
  auto kern = k_lora_gemm_pp<EPI>;
  hipError_t e = ensure_lds(kern, pp_lds(false), done);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(PP_THREADS), pp_lds(false), st, a);
  return hipGetLastError();
}
hipError_t launch_gemm_nt(int epi, const GemmArgs &a, hipStream_t st) {
  if (epi == EPI_STORE) return launch_pp<EPI_STORE>(a, st);
  if (epi == EPI_SWIGLU_FWD) return launch_pp<EPI_SWIGLU_FWD>(a, st);
  if (epi == EPI_SWIGLU_BWD) return launch_pp<EPI_SWIGLU_BWD>(a, st);
  return hipErrorInvalidValue;
}
#else
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
#endif
}  // namespace lora
