// Dense NT LoRA GEMM instantiations (eight-wave k_lora_gemm_pp): the
// forwards (store and SwiGLU epilogues) and the backward dX products that
// read a decoded, transposed copy of a 4-bit weight.
#include "gemm_launch.hpp"
#include "gemm_pp.hpp"

namespace lora {
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
// the store form over three K sources (GemmArgs::mk_*)
hipError_t launch_gemm_nt_mk(const GemmArgs &a, hipStream_t st) {
  static std::atomic<uint64_t> done{0};
  auto kern = k_lora_gemm_pp<EPI_STORE, false, true>;
  hipError_t e = ensure_lds(kern, pp_lds(false), done);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(PP_THREADS), pp_lds(false), st, a);
  return hipGetLastError();
}
hipError_t launch_gemm_nt(int epi, const GemmArgs &a, hipStream_t st) {
  if (epi == EPI_STORE) return launch_pp<EPI_STORE>(a, st);
  if (epi == EPI_STORE_NORM) return launch_pp<EPI_STORE_NORM>(a, st);
  if (epi == EPI_SWIGLU_FWD) return launch_pp<EPI_SWIGLU_FWD>(a, st);
  if (epi == EPI_SWIGLU_FWD_NORM) return launch_pp<EPI_SWIGLU_FWD_NORM>(a, st);
  if (epi == EPI_SWIGLU_BWD) return launch_pp<EPI_SWIGLU_BWD>(a, st);
  if (epi == EPI_SWIGLU_BWD_RANK) return launch_pp<EPI_SWIGLU_BWD_RANK>(a, st);
  return hipErrorInvalidValue;
}
}  // namespace lora
