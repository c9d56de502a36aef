// LoRA GEMM instantiations for the B_NN operand form.
#include "gemm_launch.hpp"
#include "gemm_pp.hpp"

// 1: the eight-wave ping-pong kernel (default); 0: the four-wave kernel
#ifndef LORA_GEMM_PP
#define LORA_GEMM_PP 1
#endif

namespace lora {
#if LORA_GEMM_PP
template <int EPI>
static hipError_t launch_pp_nn(const GemmArgs &a, hipStream_t st) {
  static std::atomic<uint64_t> done{0};
  auto kern = k_lora_gemm_pp<EPI, true>;
  hipError_t e = ensure_lds(kern, pp_lds(true), done);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(PP_THREADS), pp_lds(true), st, a);
  return hipGetLastError();
}
hipError_t launch_gemm_nn(int epi, const GemmArgs &a, hipStream_t st) {
  if (epi == EPI_STORE) return launch_pp_nn<EPI_STORE>(a, st);
  if (epi == EPI_SWIGLU_BWD) return launch_pp_nn<EPI_SWIGLU_BWD>(a, st);
  return hipErrorInvalidValue;
}
#else
hipError_t launch_gemm_nn(int epi, const GemmArgs &a, hipStream_t st) {
  if (epi == EPI_STORE) return launch_gemm_t<B_NN, EPI_STORE>(a, st);
  if (epi == EPI_SWIGLU_BWD) return launch_gemm_t<B_NN, EPI_SWIGLU_BWD>(a, st);
  return hipErrorInvalidValue;
}
#endif
}  // namespace lora
