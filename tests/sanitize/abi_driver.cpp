// Host-side driver for the AddressSanitizer / UndefinedBehaviorSanitizer run
// of liblora's C ABI (no GPU needed): every entry point is called with
// arguments that fail validation, which must return the documented status
// before any HIP call, and the workspace planners are evaluated over a grid
// of shapes up to the documented limits (size arithmetic in 64 bits, no
// overflow).  Exit status 0 = every check held.
#include <cstdio>
#include <cstdint>
#include <cstring>

#include "liblora.h"

static int failures = 0;
#define EXPECT(expr, want)                                                       \
  do {                                                                          \
    const long long got_ = (long long)(expr);                                   \
    if (got_ != (long long)(want)) {                                            \
      std::fprintf(stderr, "%s:%d: %s = %lld, expected %lld\n", __FILE__, __LINE__, \
                   #expr, got_, (long long)(want));                             \
      ++failures;                                                               \
    }                                                                           \
  } while (0)

int main() {
  // aligned fake device addresses: validation never dereferences them
  void *P = (void *)(uintptr_t)0x100000, *MIS = (void *)(uintptr_t)0x100002;
  lora_weight W;
  std::memset(&W, 0, sizeof W);
  W.fmt = LORA_W_DENSE;
  W.w = P;
  lora_weight Q = W;
  Q.fmt = LORA_W_Q4; Q.blocksize = 64; Q.w = nullptr;
  Q.codes = (const uint8_t *)P; Q.absmax = (const float *)P; Q.codebook = (const float *)P;

  EXPECT(lora_abi_version(), LORA_ABI_VERSION);
  for (int s = -1; s < 9; ++s) EXPECT(lora_strerror(s) != nullptr, 1);

  // linear forward / backward
  EXPECT(lora_linear_fwd(LORA_BF16, 16, 64, 64, 8, 16.f, nullptr, &W, P, P, P, P, 1 << 30, nullptr), LORA_ERR_NULL_POINTER);
  EXPECT(lora_linear_fwd(LORA_BF16, 16, 60, 64, 8, 16.f, P, &W, P, P, P, P, 1 << 30, nullptr), LORA_ERR_BAD_SHAPE);
  EXPECT(lora_linear_fwd(LORA_BF16, 16, 64, 64, 129, 16.f, P, &W, P, P, P, P, 1 << 30, nullptr), LORA_ERR_UNSUPPORTED);
  EXPECT(lora_linear_fwd(LORA_BF16, 16, 64, 64, 8, 16.f, MIS, &W, P, P, P, P, 1 << 30, nullptr), LORA_ERR_MISALIGNED);
  EXPECT(lora_linear_fwd(LORA_BF16, 16, 64, 64, 8, 16.f, P, &W, P, P, P, P, 0, nullptr), LORA_ERR_WORKSPACE);
  EXPECT(lora_linear_fwd(LORA_F32, 16, 64, 64, 8, 16.f, P, &Q, P, P, P, P, 1 << 30, nullptr), LORA_ERR_UNSUPPORTED);
  EXPECT(lora_linear_fwd(LORA_BF16, (int64_t)1 << 31, 64, 64, 8, 16.f, P, &W, P, P, P, P, 1 << 30, nullptr), LORA_ERR_BAD_SHAPE);
  EXPECT(lora_linear_fwd(LORA_BF16, 16, ((int64_t)1 << 20) + 8, 64, 8, 16.f, P, &W, P, P, P, P, 1 << 30, nullptr), LORA_ERR_BAD_SHAPE);
  EXPECT(lora_linear_bwd(LORA_BF16, 16, 64, 64, 8, 16.f, P, &W, P, P, nullptr, P, P, P, 0, P, 1 << 30, nullptr), LORA_ERR_NULL_POINTER);
  EXPECT(lora_linear_bwd(LORA_BF16, 16, 64, 64, 8, 16.f, P, &W, P, P, P, P, P, P, 4, P, 1 << 30, nullptr), LORA_ERR_UNSUPPORTED);
  EXPECT(lora_linear_bwd_noalloc(LORA_BF16, 65536, 4096, 4096, 128, 16.f, P, &W, P, P, P, P, P, P, 0, nullptr), LORA_ERR_WORKSPACE);
  EXPECT(lora_linear_bwd_noalloc(LORA_BF16, 16, 64, 64, 8, 16.f, P, &W, P, P, P, MIS, P, P, 0, nullptr), LORA_ERR_MISALIGNED);

  // MLP, fused norm, q/k/v
  EXPECT(lora_swiglu_mlp_fwd(LORA_BF16, 16, 64, 128, 8, 16.f, P, &W, P, P, &W, P, P, &W, P, P, nullptr, P, P, P, 1 << 30, nullptr), LORA_ERR_NULL_POINTER);
  EXPECT(lora_swiglu_mlp_fwd(LORA_BF16, 16, 64, 128, 8, 16.f, P, &Q, P, P, &W, P, P, &W, P, P, P, P, P, P, 1 << 30, nullptr), LORA_ERR_UNSUPPORTED);
  EXPECT(lora_swiglu_mlp_bwd(LORA_BF16, 16, 64, 128, 8, 16.f, P, &W, P, P, &W, P, P, &W, P, P, P, P, P, P, P, P, P, P, P, nullptr, P, 10, nullptr), LORA_ERR_NULL_POINTER);
  EXPECT(lora_rmsnorm_swiglu_mlp_fwd(LORA_BF16, 16, 64, 128, 8, 16.f, -1.f, P, P, &W, P, P, &W, P, P, &W, P, P, P, P, P, (float *)P, P, 1 << 30, nullptr), LORA_ERR_UNSUPPORTED);
  EXPECT(lora_rmsnorm_swiglu_mlp_fwd(LORA_BF16, 16, 64, 128, 8, 16.f, 1e-5f, P, nullptr, &W, P, P, &W, P, P, &W, P, P, P, P, P, (float *)P, P, 1 << 30, nullptr), LORA_ERR_NULL_POINTER);
  EXPECT(lora_rmsnorm_swiglu_mlp_bwd(LORA_BF16, 16, 64, 128, 8, 16.f, P, P, (const float *)P, &W, P, P, &W, P, P, &W, P, P, P, P, P, P, P, P, P, P, P, P, 2, P, 1 << 30, nullptr), LORA_ERR_UNSUPPORTED);
  EXPECT(lora_fold_norm_weight(LORA_BF16, 16, 60, P, P, P, nullptr), LORA_ERR_BAD_SHAPE);
  EXPECT(lora_qkv_fwd(LORA_BF16, 16, 64, 64, 32, 8, 16.f, P, &W, P, P, &W, P, P, &Q, P, P, P, P, P, P, 1 << 30, nullptr), LORA_ERR_UNSUPPORTED);
  EXPECT(lora_qkv_bwd(LORA_BF16, 16, 64, 64, 32, 8, 16.f, P, &W, P, P, &W, P, P, &W, P, P, P, P, nullptr, P, P, P, P, P, P, P, 0, P, 1 << 30, nullptr), LORA_ERR_NULL_POINTER);

  // RMSNorm folded into the q/k/v projections: bf16, dense, the stacked GEMM's shapes
  EXPECT(lora_rmsnorm_qkv_fwd(LORA_BF16, 16, 64, 256, 136, 8, 16.f, 1e-5f, P, P, &W, P, P, &W, P, P, &W, P, P, P, P, P, (float *)P, P, 1 << 30, nullptr), LORA_ERR_UNSUPPORTED);
  EXPECT(lora_rmsnorm_qkv_fwd(LORA_BF16, 16, 64, 256, 256, 8, 16.f, 1e-5f, P, P, &Q, P, P, &Q, P, P, &Q, P, P, P, P, P, (float *)P, P, 1 << 30, nullptr), LORA_ERR_UNSUPPORTED);
  EXPECT(lora_rmsnorm_qkv_fwd(LORA_BF16, 16, 64, 256, 256, 8, 16.f, 1e-5f, P, P, &W, P, P, &W, P, P, &W, P, P, P, P, P, nullptr, P, 1 << 30, nullptr), LORA_ERR_NULL_POINTER);
  EXPECT(lora_rmsnorm_qkv_fwd(LORA_BF16, 16, 64, 256, 256, 8, 16.f, 1e-5f, P, P, &W, P, P, &W, P, P, &W, P, P, P, P, P, (float *)P, P, 16, nullptr), LORA_ERR_WORKSPACE);
  EXPECT(lora_rmsnorm_qkv_bwd(LORA_BF16, 16, 64, 256, 256, 8, 16.f, P, P, (const float *)P, &W, P, P, &W, P, P, &W, P, P, P, P, P, P, P, P, P, P, P, P, 2, P, 1 << 30, nullptr), LORA_ERR_UNSUPPORTED);
  EXPECT(lora_rmsnorm_qkv_bwd(LORA_BF16, 16, 64, 256, 256, 8, 16.f, P, P, nullptr, &W, P, P, &W, P, P, &W, P, P, P, P, P, P, P, P, P, P, P, P, 0, P, 1 << 30, nullptr), LORA_ERR_NULL_POINTER);

  // standalone kernels
  EXPECT(lora_dequant4(16, 60, (const uint8_t *)P, (const float *)P, (const float *)P, 64, LORA_BF16, P, nullptr), LORA_ERR_BAD_SHAPE);
  EXPECT(lora_decode_weight(16, 64, &W, LORA_BF16, P, nullptr), LORA_ERR_UNSUPPORTED);
  EXPECT(lora_merge(LORA_BF16, 16, 64, 8, 16.f, 2, &W, P, P, P, nullptr), LORA_ERR_UNSUPPORTED);
  EXPECT(lora_rmsnorm_fwd(LORA_BF16, 16, 60, 1e-5f, P, P, P, (float *)P, nullptr), LORA_ERR_BAD_SHAPE);
  EXPECT(lora_rmsnorm_bwd(LORA_BF16, 16, 64, P, P, (const float *)P, P, P, 8, nullptr), LORA_ERR_UNSUPPORTED);

  // workspace planners over a grid of shapes up to the limits
  const int64_t Ts[] = {0, 1, 63, 64, 65, 255, 256, 8192, 16384, (int64_t)1 << 20, (int64_t)1 << 30};
  const int64_t Ks[] = {8, 64, 72, 4096, 14336, (int64_t)1 << 20};
  const int64_t Rs[] = {1, 3, 16, 17, 64, 128};
  size_t checked = 0;
  for (int64_t T : Ts)
    for (int64_t k : Ks)
      for (int64_t n : Ks)
        for (int64_t r : Rs)
          for (int op = 0; op <= LORA_OP_RMSNORM_QKV_BWD; ++op)
            for (int dt = 0; dt < 2; ++dt)
              for (int wf = 0; wf < 3; ++wf) {
                const size_t fast = lora_workspace_bytes(op, dt, wf, T, k, n, r);
                const size_t mini = lora_workspace_bytes(op | LORA_WS_MINIMAL, dt, wf, T, k, n, r);
                if (op == LORA_OP_RMSNORM_QKV_FWD || op == LORA_OP_RMSNORM_QKV_BWD) {
                  EXPECT(fast, 0);
                  EXPECT(mini, 0);
                  const size_t q = lora_qkv_workspace_bytes(op, dt, wf, T, k, n, n, r);
                  // one strategy: the minimal flag asks for the same size
                  EXPECT(lora_qkv_workspace_bytes(op | LORA_WS_MINIMAL, dt, wf, T, k, n, n, r), q);
                  if (q) EXPECT(dt == LORA_BF16 && wf == LORA_W_DENSE, 1);
                } else if (op == LORA_OP_QKV_FWD || op == LORA_OP_QKV_BWD) {
                  EXPECT(fast, 0);   // lora_qkv_workspace_bytes answers those
                  const size_t q = lora_qkv_workspace_bytes(op, dt, wf, T, k, n, n / 2 + 8, r);
                  const size_t qm = lora_qkv_workspace_bytes(op | LORA_WS_MINIMAL, dt, wf, T, k, n, n / 2 + 8, r);
                  if (qm > q) EXPECT(qm <= q, 1);
                } else if (mini > fast) {
                  EXPECT(mini <= fast, 1);   // the minimal strategy never needs more
                }
                ++checked;
              }
  EXPECT(lora_workspace_bytes(LORA_OP_MLP_FWD, LORA_BF16, 0, -1, 64, 64, 8), 0);
  EXPECT(lora_workspace_bytes(0x4000, LORA_BF16, 0, 16, 64, 64, 8), 0);
  std::printf("abi driver: %zu planner cases, %d failures\n", checked, failures);
  return failures ? 1 : 0;
}
