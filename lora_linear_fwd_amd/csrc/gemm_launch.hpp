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

template <int BMODE, int EPI, int PF = 0>
inline hipError_t launch_gemm_t(const GemmArgs &a, hipStream_t st) {
  static std::atomic<uint64_t> done{0};
  constexpr int BK = gemm_bk<BMODE>(), NS = gemm_nstage<BMODE>();
  constexpr size_t lds = gemm_lds_bytes<BMODE, PF, BK, NS>();
  auto kern = k_lora_gemm<BMODE, EPI, PF, BK, NS>;
  hipError_t e = ensure_lds(kern, lds, done);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)(a.tiles_m * a.tiles_n);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHREADS), lds, st, a);
  return hipGetLastError();
}

// dense NT with a K step of 64: loops of at least this many K elements also
// prefetch one step further into L2 (measured: helps K = 14336 and 28672,
// hurts K = 4096); the K-step-32 pipeline runs three steps ahead instead
constexpr int kPrefetchMinK = 8192;
constexpr bool kNtPrefetch = gemm_bk<B_NT>() == 64;
hipError_t launch_gemm_nt(int epi, const GemmArgs &a, hipStream_t st);
hipError_t launch_gemm_nt_q4(int epi, const GemmArgs &a, hipStream_t st);
hipError_t launch_gemm_nn(int epi, const GemmArgs &a, hipStream_t st);
hipError_t launch_gemm_nn_q4(int epi, const GemmArgs &a, hipStream_t st);
hipError_t launch_gemm_nt_q4dq(int epi, const GemmArgs &a, hipStream_t st);
hipError_t launch_gemm_nn_q4dq(int epi, const GemmArgs &a, hipStream_t st);

}  // namespace lora
