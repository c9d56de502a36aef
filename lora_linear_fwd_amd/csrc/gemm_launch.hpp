// Instantiation + launch of the LoRA GEMM for one B-operand form.
#pragma once
#include <atomic>
#include "gemm_lora.hpp"

namespace lora {

// Raise the dynamic-LDS limit of a kernel once per device (the kernels need
// more than the 64 KB default).
template <typename Kern>
inline hipError_t ensure_lds(Kern kern, size_t bytes, std::atomic<uint64_t> &done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// the four-wave kernel with a 4-bit weight decoded in its LDS fill
template <int BMODE, int EPI>
inline hipError_t launch_gemm_t(const GemmArgs &a, hipStream_t st) {
  static std::atomic<uint64_t> done{0};
  constexpr size_t lds = gemm_lds_bytes<BMODE>();
  auto kern = k_lora_gemm<BMODE, EPI>;
  hipError_t e = ensure_lds(kern, lds, done);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHREADS), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_gemm_nt(int epi, const GemmArgs &a, hipStream_t st);
hipError_t launch_gemm_nt_mk(const GemmArgs &a, hipStream_t st);
hipError_t launch_gemm_nt_q4(int epi, const GemmArgs &a, hipStream_t st);
hipError_t launch_gemm_nn(int epi, const GemmArgs &a, hipStream_t st);
hipError_t launch_gemm_nn_q4(int epi, const GemmArgs &a, hipStream_t st);
hipError_t launch_gemm_nt_q4dq(int epi, const GemmArgs &a, hipStream_t st);
hipError_t launch_gemm_nn_q4dq(int epi, const GemmArgs &a, hipStream_t st);

}  // namespace lora
