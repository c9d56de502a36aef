// Dense NN LoRA GEMM instantiations (eight-wave k_lora_gemm_pp reading the
// weight as stored): the backward dX products, with the store and SwiGLU'
// epilogues.
#include "gemm_launch.hpp"
#include "gemm_pp.hpp"

namespace lora {
template <int EPI>
static hipError_t launch_pp_nn(const GemmArgs &a, hipStream_t st) {
  static std::atomic<uint64_t> done{0};
  auto kern = k_lora_gemm_pp<EPI, true>;
  // the rank-r SwiGLU' epilogue stages 20 KB per wave
  constexpr size_t lds = EPI == EPI_SWIGLU_BWD_RANK ? pp_lds(false) : pp_lds(true);
  hipError_t e = ensure_lds(kern, lds, done);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(PP_THREADS), lds, st, a);
  return hipGetLastError();
}
hipError_t launch_gemm_nn(int epi, const GemmArgs &a, hipStream_t st) {
  if (epi == EPI_STORE) return launch_pp_nn<EPI_STORE>(a, st);
  if (epi == EPI_STORE_NORM) return launch_pp_nn<EPI_STORE_NORM>(a, st);
  if (epi == EPI_SWIGLU_BWD) return launch_pp_nn<EPI_SWIGLU_BWD>(a, st);
  if (epi == EPI_SWIGLU_BWD_RANK) return launch_pp_nn<EPI_SWIGLU_BWD_RANK>(a, st);
  return hipErrorInvalidValue;
}
}  // namespace lora
