// liblora C ABI: argument validation, workspace planning and kernel dispatch.
// Every check runs before the first HIP call; no exception leaves this file.
#include "liblora.h"
#ifdef LORA_TIMING_HOOKS
#include "liblora_timing.h"
#endif

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <initializer_list>

#include "aux_kernels.hpp"
#include "gemm_launch.hpp"
#include "norm_kernels.hpp"

using namespace lora;

namespace {


inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
constexpr int64_t kMaxFeatures = (int64_t)1 << 20;
constexpr int kMaxDevices = 64;
inline int rs_of(int64_t width) { return (int)(cdiv(width, 16) * 16); }
inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// ---------------------------------------------------------------- workspace
struct Bump {
  size_t cur = 0;
  size_t take(size_t bytes) {
    const size_t o = cur;
    cur += (bytes + 255) & ~(size_t)255;
    return o;
  }
};

// split choices shared by the planner and the launchers
struct NTSplit { int ks; int kchunk; };
// Token block of the skinny NT kernel: from 64 rank columns on, 128 tokens in
// eight waves, which halves the side tile's re-reads per Z byte at the same
// per-wave registers; 64 tokens in four waves for narrower ranks.
constexpr int nt_tb(int RS) { return RS >= 64 ? 128 : 64; }
// K chunks so that the grid about fills the workgroups resident at once for
// the rank width: four 64-token workgroups per CU below 64 rank columns, two
// 128-token ones up to 144 and one from 160 (the accumulators' registers)
inline NTSplit nt_split(int64_t T, int64_t K, int RS) {
  const int64_t gx = std::max<int64_t>(1, cdiv(T, nt_tb(RS)));
  const int64_t slots = RS < 64 ? 1024 : (RS < 160 ? 512 : 256);
  // at most one round of resident workgroups: a second round that holds a
  // few workgroups would take as long as the first
  int64_t ks = std::max<int64_t>(1, std::min<int64_t>(slots / gx, cdiv(K, 512)));
  int64_t kchunk = cdiv(cdiv(K, ks), 128) * 128;
  ks = std::max<int64_t>(1, cdiv(K, kchunk));
  return {(int)ks, (int)kchunk};
}
struct TNSplit { int ts; int tchunk; };
// Token chunks so that the grid about fills the workgroups resident at once:
// four per CU for the narrowest ranks, fewer as the accumulators take more
// of the register file (three from 32 rank columns, two from 64, one from 128)
inline TNSplit tn_split(int64_t T, int64_t N, int RS) {
  const int64_t gx = cdiv(N, 256);
  const int64_t slots = RS >= 128 ? 256 : (RS >= 64 ? 512 : (RS >= 32 ? 768 : 1024));
  // at most one round of resident workgroups (as for the NT split)
  int64_t ts = std::max<int64_t>(1, std::min<int64_t>(slots / gx, cdiv(T, 64)));
  int64_t tchunk = std::max<int64_t>(64, cdiv(cdiv(T, ts), 64) * 64);
  ts = std::max<int64_t>(1, cdiv(T, tchunk));
  return {(int)ts, (int)tchunk};
}
inline size_t nt_part_bytes(int64_t T, int64_t K, int RS) {
  return (size_t)nt_split(T, K, RS).ks * T * RS * 4;
}
inline size_t tn_part_bytes(int64_t T, int64_t N, int RS) {
  return (size_t)tn_split(T, N, RS).ts * RS * N * 4;
}
// dual pass: 256-column blocks per segment x token chunks (multiples of 64)
struct DualSplit { int nb0, nb1, ts, tchunk; };
// Fill the workgroups resident at once (three per CU for the 16-wide pass
// over a stored operand, two otherwise: registers and LDS) in one round
// rather than spill a partial second round
inline int64_t dual_slots(int RS, bool zswiglu) { return RS <= 16 && !zswiglu ? 768 : 512; }
inline DualSplit dual_split(int64_t T, int64_t N, int64_t nsplit, int64_t slots) {
  DualSplit d;
  d.nb0 = (int)cdiv(nsplit, 256);
  d.nb1 = (int)cdiv(N - nsplit, 256);
  const int64_t nbc = std::max<int64_t>(1, d.nb0 + d.nb1);
  int64_t ts = std::max<int64_t>(1, std::min<int64_t>(cdiv(T, 64), slots / nbc));
  const int64_t tchunk = std::max<int64_t>(64, cdiv(cdiv(T, ts), 64) * 64);
  d.tchunk = (int)tchunk;
  d.ts = (int)std::max<int64_t>(1, cdiv(T, tchunk));
  return d;
}
inline size_t dual_u_bytes(int64_t T, int64_t N, int64_t nsplit, int RS) {
  const DualSplit d = dual_split(T, N, nsplit, dual_slots(RS, false));
  return (size_t)(d.nb0 + d.nb1) * T * RS * 4;
}
inline size_t dual_v_bytes(int64_t T, int64_t N, int64_t nsplit, int RS) {
  // the larger slot count of the two forms: the most token chunks
  return (size_t)dual_split(T, N, nsplit, dual_slots(RS, false)).ts * RS * N * 4;
}
inline int64_t ldp_of(int64_t T) { return std::max<int64_t>(64, cdiv(T, 64) * 64); }

// `wcopy`: room for a bf16 copy of the base weight (decoded or transposed)
struct LinFwdPlan { size_t side, epi, hpart, hbf, wbuf, total; };
LinFwdPlan plan_lin_fwd(int64_t T, int64_t k, int64_t n, int64_t r, bool wcopy) {
  Bump b; LinFwdPlan p{};
  const int RS = rs_of(r);
  if (wcopy) p.wbuf = b.take((size_t)n * k * 2);
  p.side = b.take((size_t)RS * k * 2);
  p.epi = b.take((size_t)n * RS * 2);
  p.hpart = b.take(nt_part_bytes(T, k, RS));
  p.hbf = b.take((size_t)T * RS * 2);
  p.total = b.cur;
  return p;
}

struct LinBwdPlan { size_t side_nn, epi_nn, side_nt, g32, gbf, h32, ntpart, tnpart, wbuf, total; };
LinBwdPlan plan_lin_bwd(int64_t T, int64_t k, int64_t n, int64_t r, bool wcopy) {
  Bump b; LinBwdPlan p{};
  const int RS = rs_of(r);
  if (wcopy) p.wbuf = b.take((size_t)k * n * 2);
  p.side_nn = b.take((size_t)RS * n * 2);
  p.epi_nn = b.take((size_t)k * RS * 2);
  p.side_nt = b.take((size_t)RS * k * 2);
  p.g32 = b.take((size_t)T * RS * 4);
  p.gbf = b.take((size_t)T * RS * 2);
  p.h32 = b.take((size_t)T * RS * 4);
  p.ntpart = b.take(std::max(nt_part_bytes(T, n, RS), nt_part_bytes(T, k, RS)));
  p.tnpart = b.take(std::max(tn_part_bytes(T, k, RS), tn_part_bytes(T, n, RS)));
  p.total = b.cur;
  return p;
}

// The gate/up forward's SwiGLU epilogue forms H_d = h Ad^T as per-tile
// partials (one 16-wide MFMA block of rank) when it runs in the eight-wave
// kernel, instead of a separate pass over h
inline bool mlp_fwd_hd_fused(int64_t r) { return rs_of(r) == 16; }
inline int64_t gu_tiles_n(int64_t f) { return cdiv(f, 128); }
struct MlpFwdPlan { size_t h, side_gu, epi_gu, side_d, epi_d, hpart, hbf, wbuf, total; };
// hd: H_d from the gate/up epilogue; its partials [gu_tiles_n(f) x T x 16]
// fp32 share hpart with the pass over X, which is done by then
MlpFwdPlan plan_mlp_fwd(int64_t T, int64_t d, int64_t f, int64_t r, bool wcopy, bool hd) {
  Bump b; MlpFwdPlan p{};
  const int RS1 = rs_of(2 * r), RS2 = rs_of(r);
  if (wcopy) p.wbuf = b.take((size_t)2 * f * d * 2);   // Wg | Wu, later Wd
  p.h = b.take((size_t)T * f * 2);
  p.side_gu = b.take((size_t)RS1 * d * 2);
  p.epi_gu = b.take((size_t)2 * f * RS1 * 2);
  p.side_d = b.take((size_t)RS2 * f * 2);
  p.epi_d = b.take((size_t)d * RS2 * 2);
  p.hpart = b.take(std::max(nt_part_bytes(T, d, RS1),
                            hd ? (size_t)gu_tiles_n(f) * T * 16 * 4 : nt_part_bytes(T, f, RS2)));
  p.hbf = b.take((size_t)T * std::max(RS1, RS2) * 2);
  p.total = b.cur;
  return p;
}

// The dual rank-r pass is used up to RS = 32 (2r rounded): its per-column-
// block partials grow with RS, and at r = 64 they outweigh the second read it
// saves (measured: 0.97 ms vs 0.5 ms per step at T = 16384).
inline bool mlp_bwd_dual(int64_t r) { return rs_of(r) <= 32; }
struct MlpBwdPlan {
  size_t de, dg, side_d_nn, epi_d_nn, side_d_nt, epi_gu_nn, side_gu_nt, side_gu_nn;
  size_t side_g, side_u, pt_d, pt_g, pt_u, part_u, part_v;
  size_t gd32, gdbf, hd32, ggu32, ggubf, hgu32, ntpart, tnpart, wbuf, cpart, nkk;
  size_t fu_d, fu_gu, fv_d, fv_gu;   // per-tile partials of the rank-fused SwiGLU' GEMM
  size_t hsv;                        // h = silu(e) g from the SwiGLU' epilogue (wide ranks)
  size_t total;
};
// The down-projection backward forms the four rank-r products of the
// backward in its SwiGLU' epilogue (EPI_SWIGLU_BWD_RANK) when the rank fits
// one 16-wide MFMA block
inline bool mlp_bwd_rank_fused(int64_t r) { return rs_of(r) == 16; }
// Wide ranks (separate rank-r passes) with the eight-wave down backward: its
// SwiGLU' epilogue also writes h, which the two passes for H_d and dAd then
// read instead of e and g (half the bytes, no recomputation)
inline bool mlp_bwd_hsave(int64_t r, bool eight_wave) { return !mlp_bwd_dual(r) && eight_wave; }
// Wide ranks that fill whole 16-column groups: G_gu and dBg, dBu are
// block-diagonal in the rank (de pairs with Bg and H_g, dg with Bu and H_u),
// so they run as two r-wide passes instead of one 2r-wide pass over [de | dg]
inline bool mlp_bwd_gu_segmented(int64_t r) { return !mlp_bwd_dual(r) && r % 16 == 0; }
MlpBwdPlan plan_mlp_bwd(int64_t T, int64_t d, int64_t f, int64_t r, bool wcopy, bool norm = false,
                        bool hsave = false) {
  Bump b; MlpBwdPlan p{};
  if (norm) {   // folded RMSNorm: row partials per 64-column block of the down backward
    p.cpart = b.take((size_t)cdiv(f, 256) * 4 * T * 4);
    p.nkk = b.take((size_t)T * 4);
  }
  const int RS1 = rs_of(2 * r), RS2 = rs_of(r);
  if (wcopy) p.wbuf = b.take((size_t)2 * d * f * 2);   // Wd^T, later [Wg^T | Wu^T]
  // de and dg interleaved as one [T x 2f] matrix (dg = de + f): the dX
  // GEMM then reads [de | dg] as one operand with tile-local offsets
  p.de = b.take((size_t)T * 2 * f * 2);
  p.dg = p.de + (size_t)f * 2;
  p.side_d_nn = b.take((size_t)RS2 * d * 2);
  p.epi_d_nn = b.take((size_t)f * RS2 * 2);
  p.side_d_nt = b.take((size_t)RS2 * f * 2);
  p.epi_gu_nn = b.take((size_t)d * RS1 * 2);
  p.side_gu_nt = b.take((size_t)RS1 * d * 2);
  p.gd32 = b.take((size_t)T * RS2 * 4);
  p.gdbf = b.take((size_t)T * RS2 * 2);
  p.hd32 = b.take((size_t)T * RS2 * 4);
  p.ggu32 = b.take((size_t)T * RS1 * 4);
  p.ggubf = b.take((size_t)T * RS1 * 2);
  p.hgu32 = b.take((size_t)T * RS1 * 4);
  if (mlp_bwd_dual(r)) {
    p.ntpart = b.take(std::max(nt_part_bytes(T, d, RS2), nt_part_bytes(T, d, RS1)));
    p.tnpart = b.take(std::max(tn_part_bytes(T, d, RS2), tn_part_bytes(T, d, RS1)));
    p.side_g = b.take((size_t)RS2 * f * 2);
    p.side_u = b.take((size_t)RS2 * f * 2);
    const size_t ptb = (size_t)RS2 * ldp_of(T) * 2;
    p.pt_d = b.take(ptb);
    p.pt_g = b.take(ptb);
    p.pt_u = b.take(ptb);
    p.part_u = b.take(std::max(dual_u_bytes(T, f, f, RS2), dual_u_bytes(T, 2 * f, f, RS2)));
    p.part_v = b.take(std::max(dual_v_bytes(T, f, f, RS2), dual_v_bytes(T, 2 * f, f, RS2)));
    if (mlp_bwd_rank_fused(r)) {
      const int64_t tn = cdiv(f, 256), tm = cdiv(T, 256);
      p.fu_d = b.take((size_t)tn * T * 16 * 4);
      p.fu_gu = b.take((size_t)2 * tn * T * 16 * 4);
      p.fv_d = b.take((size_t)tm * 16 * f * 4);
      p.fv_gu = b.take((size_t)tm * 16 * 2 * f * 4);
    }
  } else {
    if (hsave) p.hsv = b.take((size_t)T * f * 2);
    p.side_gu_nn = b.take((size_t)RS1 * 2 * f * 2);
    // (the r-wide passes of the segmented form are within the f-wide sizes)
    p.ntpart = b.take(std::max({nt_part_bytes(T, d, RS2), nt_part_bytes(T, d, RS1),
                                nt_part_bytes(T, f, RS2), nt_part_bytes(T, 2 * f, RS1)}));
    p.tnpart = b.take(std::max({tn_part_bytes(T, d, RS2), tn_part_bytes(T, d, RS1),
                                tn_part_bytes(T, f, RS2), tn_part_bytes(T, 2 * f, RS1)}));
  }
  p.total = b.cur;
  return p;
}

// fused q/k/v projections: N = nq + 2 nkv output columns, rank products of
// width RS3 = 3r rounded up to 16 (q, k, v blocks stacked)
inline bool qkv_rank_ok(int64_t r) { return rs_of(3 * r) <= 256; }
// shapes the stacked q/k/v GEMM takes: every tile's columns in one projection
inline bool qkv_shapes_ok(int64_t k, int64_t nq, int64_t nkv, int64_t r) {
  return r > 0 && r <= LORA_MAX_RANK && qkv_rank_ok(r) && k > 0 && nq > 0 && nkv > 0 &&
         nq % BN == 0 && nkv % BN == 0 && k <= kMaxFeatures && nq + 2 * nkv <= kMaxFeatures;
}
struct QkvFwdPlan { size_t side, epi, hpart, hbf, wbuf, total; };
QkvFwdPlan plan_qkv_fwd(int64_t T, int64_t k, int64_t nq, int64_t nkv, int64_t r, bool wcopy) {
  Bump b; QkvFwdPlan p{};
  const int64_t N = nq + 2 * nkv;
  const int RS3 = rs_of(3 * r);
  if (wcopy) p.wbuf = b.take((size_t)N * k * 2);
  p.side = b.take((size_t)RS3 * k * 2);
  p.epi = b.take((size_t)N * RS3 * 2);
  p.hpart = b.take(nt_part_bytes(T, k, RS3));
  p.hbf = b.take((size_t)T * RS3 * 2);
  p.total = b.cur;
  return p;
}
struct QkvBwdPlan { size_t dyc, side_nn, epi_nn, side_nt, g32, gbf, h32, ntpart, tnpart, wbuf, gn, total; };
// The products with dQ, dK, dV (G and dB) are block-diagonal in the rank:
// with r a multiple of 16 each block is its own rank-r pass over its own
// gradient (a third of the contraction work of one 3r-wide pass each, and no
// packed [dQ | dK | dV] for them)
inline bool qkv_bwd_segmented(int64_t r) { return r % 16 == 0; }
// norm: an RMSNorm folded into the projections (lora_rmsnorm_qkv_bwd) adds a
// [T x k] bf16 buffer for the projections' input gradient
QkvBwdPlan plan_qkv_bwd(int64_t T, int64_t k, int64_t nq, int64_t nkv, int64_t r,
                        bool norm = false) {
  Bump b; QkvBwdPlan p{};
  const int64_t N = nq + 2 * nkv;
  const int RS3 = rs_of(3 * r);
  p.wbuf = b.take((size_t)k * N * 2);
  if (norm) p.gn = b.take((size_t)T * k * 2);
  p.dyc = b.take((size_t)T * N * 2);
  p.side_nn = b.take((size_t)RS3 * N * 2);
  p.epi_nn = b.take((size_t)k * RS3 * 2);
  p.side_nt = b.take((size_t)RS3 * k * 2);
  p.g32 = b.take((size_t)T * RS3 * 4);
  p.gbf = b.take((size_t)T * RS3 * 2);
  p.h32 = b.take((size_t)T * RS3 * 4);
  size_t ntb = std::max(nt_part_bytes(T, N, RS3), nt_part_bytes(T, k, RS3));
  size_t tnb = std::max(tn_part_bytes(T, k, RS3), tn_part_bytes(T, N, RS3));
  if (qkv_bwd_segmented(r)) {
    ntb = std::max({ntb, nt_part_bytes(T, nq, (int)r), nt_part_bytes(T, nkv, (int)r)});
    tnb = std::max({tnb, tn_part_bytes(T, nq, (int)r), tn_part_bytes(T, nkv, (int)r)});
  }
  p.ntpart = b.take(ntb);
  p.tnpart = b.take(tnb);
  p.total = b.cur;
  return p;
}

// fp32 path workspaces
size_t plan_f32(int op, int64_t T, int64_t kd, int64_t nf, int64_t r) {
  switch (op) {
    case LORA_OP_LINEAR_FWD: return (size_t)T * r * 4;
    case LORA_OP_LINEAR_BWD: return 2 * (size_t)T * r * 4;
    case LORA_OP_MLP_FWD: return (size_t)T * nf * 4 + (size_t)T * r * 4 + 256;
    case LORA_OP_MLP_BWD: return 4 * (size_t)T * nf * 4 + 2 * (size_t)T * r * 4 + 1024;
  }
  return 0;
}

// ------------------------------------------------------------- validation
struct WeightView {
  bool q4;                // Q4 or Q4_DQ
  int fmt;                // lora_wfmt
  const bf16_t *w;
  const uint8_t *codes;
  AbsmaxSrc absmax;       // plain or double-quantised block constants
  const float *codebook;
  const bf16_t *wt;       // dense, optional: W^T [k x n] kept by the caller
};

int check_weight(const lora_weight *W, int dtype, int64_t k_in, WeightView &out) {
  if (!W) return LORA_ERR_NULL_POINTER;
  if (W->fmt == LORA_W_DENSE) {
    if (!W->w) return LORA_ERR_NULL_POINTER;
    if (!aligned16(W->w) || (W->wt && !aligned16(W->wt))) return LORA_ERR_MISALIGNED;
    // the transposed copy serves the bf16 GEMMs only
    const bf16_t *wt = dtype == LORA_BF16 ? (const bf16_t *)W->wt : nullptr;
    out = {false, LORA_W_DENSE, (const bf16_t *)W->w, nullptr, AbsmaxSrc{}, nullptr, wt};
    return LORA_OK;
  }
  if (W->fmt != LORA_W_Q4 && W->fmt != LORA_W_Q4_DQ) return LORA_ERR_UNSUPPORTED;
  if (dtype != LORA_BF16) return LORA_ERR_UNSUPPORTED;
  if (W->blocksize != 64) return LORA_ERR_UNSUPPORTED;
  if (!W->codes || !W->codebook) return LORA_ERR_NULL_POINTER;
  if (k_in % 64) return LORA_ERR_BAD_SHAPE;
  if (!aligned16(W->codes) || !aligned16(W->codebook)) return LORA_ERR_MISALIGNED;
  AbsmaxSrc am{};
  if (W->fmt == LORA_W_Q4) {
    if (!W->absmax) return LORA_ERR_NULL_POINTER;
    if (!aligned16(W->absmax)) return LORA_ERR_MISALIGNED;
    am.absmax = W->absmax;
  } else {
    if (W->absmax_blocksize != 256) return LORA_ERR_UNSUPPORTED;
    if (!W->absmax_codes || !W->absmax_codebook || !W->absmax_scale) return LORA_ERR_NULL_POINTER;
    if (!aligned16(W->absmax_codes) || !aligned16(W->absmax_codebook) ||
        !aligned16(W->absmax_scale))
      return LORA_ERR_MISALIGNED;
    am.codes = W->absmax_codes;
    am.table = W->absmax_codebook;
    am.scale = W->absmax_scale;
    am.offset = W->absmax_offset;
  }
  out = {true, W->fmt, nullptr, W->codes, am, W->codebook, nullptr};
  return LORA_OK;
}

int check_dims(int dtype, int64_t T, int64_t k, int64_t n, int64_t r) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_UNSUPPORTED;
  if (T < 0 || k <= 0 || n <= 0 || r <= 0) return LORA_ERR_BAD_SHAPE;
  if (r > LORA_MAX_RANK) return LORA_ERR_UNSUPPORTED;
  // feature sizes up to 2^20: a GEMM tile's 256 rows of any operand then
  // span less than 2^31 bytes, the range of one buffer descriptor
  if (T > (int64_t)1 << 30 || k > kMaxFeatures || n > kMaxFeatures) return LORA_ERR_BAD_SHAPE;
  // every GEMM grid (256-token by 128- or 256-column tiles) fits a 31-bit count
  if (cdiv(T, 256) * cdiv(2 * std::max(k, n), 128) >= ((int64_t)1 << 31)) return LORA_ERR_BAD_SHAPE;
  if (dtype == LORA_BF16 && ((k % 8) || (n % 8))) return LORA_ERR_BAD_SHAPE;
  return LORA_OK;
}

int check_ptrs(std::initializer_list<const void *> ps) {
  for (const void *p : ps)
    if (!p) return LORA_ERR_NULL_POINTER;
  for (const void *p : ps)
    if (!aligned16(p)) return LORA_ERR_MISALIGNED;
  return LORA_OK;
}

// token-sized tensors ([T x ...]) hold no elements when T == 0 and may then
// be NULL
int check_tok_ptrs(int64_t T, std::initializer_list<const void *> ps) {
  if (T == 0) {
    for (const void *p : ps)
      if (p && !aligned16(p)) return LORA_ERR_MISALIGNED;
    return LORA_OK;
  }
  for (const void *p : ps)
    if (!p) return LORA_ERR_NULL_POINTER;
  for (const void *p : ps)
    if (!aligned16(p)) return LORA_ERR_MISALIGNED;
  return LORA_OK;
}

#define LORA_TRY(expr)                         \
  do {                                         \
    int _st = (expr);                          \
    if (_st != LORA_OK) return _st;            \
  } while (0)
#define HIP_TRY(expr)                          \
  do {                                         \
    if ((expr) != hipSuccess) return LORA_ERR_HIP; \
  } while (0)

inline unsigned blocks_for(int64_t count, int per = 256) { return (unsigned)cdiv(count, per); }

// ------------------------------------------------------------ bf16 helpers
// Collects the call's small operand copies (zero-padded side / epilogue
// operands, layouts as documented at k_prep) and launches them at once.
struct Prep {
  PrepBatch b{};
  unsigned blocks = 0;
  void add(int kind, bf16_t *dst, int64_t a, int64_t bb, const void *src0, const void *src1,
           int64_t r, int64_t split, int tr, const void *src2 = nullptr, int64_t split2 = 0,
           const void *cs = nullptr) {
    const int64_t cnt = a * bb;
    if (cnt == 0) return;
    PrepJob &j = b.job[b.njobs];
    j = PrepJob{dst, (const bf16_t *)src0, (const bf16_t *)src1, (const bf16_t *)src2, kind,
                (int)a, (int)bb, (int)r, (int)split, (int)split2, tr, (const bf16_t *)cs};
    b.start[b.njobs] = blocks;
    // 8 elements per thread for rows of a multiple of 8 (see k_prep)
    blocks += (unsigned)cdiv(bb % 8 == 0 ? cnt / 8 : cnt, 256);
    ++b.njobs;
  }
  // side[q][k], q < RS, k < K
  void side(bf16_t *dst, int RS, int64_t K, const void *s0, const void *s1, int64_t r,
            int64_t ksplit, int tr, const void *s2 = nullptr, int64_t ksplit2 = 0,
            const void *cs = nullptr) {
    add(0, dst, RS, K, s0, s1, r, ksplit, tr, s2, ksplit2, cs);
  }
  // epi[row][q], row < rows, q < RS
  void epi(bf16_t *dst, int64_t rows, int RS, const void *s0, const void *s1, int64_t r,
           int64_t rsplit, int tr, const void *s2 = nullptr, int64_t rsplit2 = 0,
           const void *cs = nullptr) {
    add(1, dst, rows, RS, s0, s1, r, rsplit, tr, s2, rsplit2, cs);
  }
  int launch(hipStream_t st) {
    if (!b.njobs) return LORA_OK;
    b.start[b.njobs] = blocks;
    hipLaunchKernelGGL(k_prep, dim3(blocks), dim3(256), 0, st, b);
    HIP_TRY(hipGetLastError());
    return LORA_OK;
  }
};

// out = Z . SIDE^T over all K (deterministic split-K); fp32 and/or scaled bf16
// side [RS x K] with row stride lds (0: K); outputs [T x RS] with row
// stride ldo (0: RS); with side1, side rows >= rsplit come from side1
int skinny_nt(int RS, bool zswiglu, int64_t T, int64_t K, const bf16_t *Z0, const bf16_t *Z1,
              int64_t ksplit, int64_t ldz, const bf16_t *E, const bf16_t *G, const bf16_t *side,
              float *part, float *out32, bf16_t *outbf, float scale, hipStream_t st,
              const float *rowscale = nullptr, int64_t lds = 0, int ldo = 0,
              const bf16_t *side1 = nullptr, int rsplit = 0) {
  if (T == 0) return LORA_OK;
  const NTSplit sp = nt_split(T, K, RS);
  SkinnyNTArgs a{(int)T, (int)K, (int)ksplit, sp.kchunk, Z0, Z1, ldz, E, G, side, part,
                 lds ? lds : K, side1, side1 ? rsplit : RS};
  dim3 grid((unsigned)cdiv(T, nt_tb(RS)), (unsigned)sp.ks);
#define SNT(R)                                                                    \
  case R:                                                                         \
    if (zswiglu)                                                                  \
      hipLaunchKernelGGL((k_skinny_nt<R, true, nt_tb(R)>), grid, dim3(nt_tb(R) * 4), 0, st, a); \
    else                                                                          \
      hipLaunchKernelGGL((k_skinny_nt<R, false, nt_tb(R)>), grid, dim3(nt_tb(R) * 4), 0, st, a); \
    break;
  switch (RS) {
    SNT(16) SNT(32) SNT(48) SNT(64) SNT(80) SNT(96) SNT(112) SNT(128)
    SNT(144) SNT(160) SNT(176) SNT(192) SNT(208) SNT(224) SNT(240) SNT(256)
    default: return LORA_ERR_UNSUPPORTED;
  }
#undef SNT
  HIP_TRY(hipGetLastError());
  const int64_t cnt = T * RS;
  hipLaunchKernelGGL(k_reduce_side, dim3(blocks_for(cnt)), dim3(256), 0, st, part, sp.ks, cnt,
                     scale, out32, outbf, rowscale, RS, ldo ? ldo : RS);
  HIP_TRY(hipGetLastError());
  return LORA_OK;
}

// adapter gradient: s * P^T Z reduced over T, scattered per ReduceTNArgs
int skinny_tn(int RS, bool zswiglu, int64_t T, int64_t N, const float *P, const bf16_t *Z0,
              const bf16_t *Z1, int64_t nsplit, int64_t ldz, const bf16_t *E, const bf16_t *G,
              float *part, int64_t r, float scale, int transposed, bf16_t *out0, bf16_t *out1,
              int64_t out_nsplit, hipStream_t st, bf16_t *out2 = nullptr,
              int64_t out_nsplit2 = 0, const bf16_t *colscale = nullptr, int64_t ldp = 0) {
  const TNSplit sp = tn_split(T, N, RS);
  SkinnyTNArgs a{(int)T, (int)N, (int)nsplit, sp.tchunk, P, Z0, Z1, ldz, E, G, part,
                 ldp ? ldp : RS};
  dim3 grid((unsigned)cdiv(N, 256), (unsigned)sp.ts);
#define STN(R)                                                                          \
  case R:                                                                               \
    if (zswiglu) hipLaunchKernelGGL((k_skinny_tn<R, true>), grid, dim3(256), 0, st, a);  \
    else hipLaunchKernelGGL((k_skinny_tn<R, false>), grid, dim3(256), 0, st, a);         \
    break;
  switch (RS) {
    STN(16) STN(32) STN(48) STN(64) STN(80) STN(96) STN(112) STN(128)
    STN(144) STN(160) STN(176) STN(192) STN(208) STN(224) STN(240) STN(256)
    default: return LORA_ERR_UNSUPPORTED;
  }
#undef STN
  HIP_TRY(hipGetLastError());
  ReduceTNArgs ra{part,       sp.ts, RS, (int)N, (int)r, (int)out_nsplit, scale, transposed, out0,
                  out1,       (int)r, out2, (int)out_nsplit2, (int)(2 * r), colscale};
  hipLaunchKernelGGL(k_reduce_tn, dim3(blocks_for((int64_t)RS * N)), dim3(256), 0, st, ra);
  HIP_TRY(hipGetLastError());
  return LORA_OK;
}

// bf16 copies of a base weight W [rows x cols] in the workspace
//   decode_w:    out = W (4-bit codes decoded), same layout
//   transpose_w: out[c * ld_out + r] = W[r][c] (decoded if 4-bit)
int decode_w(bf16_t *out, const WeightView &w, int64_t rows, int64_t cols, hipStream_t st) {
  const int64_t total = rows * cols;
  hipLaunchKernelGGL(k_dequant4, dim3(blocks_for(total / 32)), dim3(256), 0, st, w.codes,
                     w.absmax, w.codebook, total, out);
  HIP_TRY(hipGetLastError());
  return LORA_OK;
}
int transpose_w(bf16_t *out, int64_t ld_out, const WeightView &w, int64_t rows, int64_t cols,
                hipStream_t st) {
  const int64_t rb = cdiv(rows, 256), cb = cdiv(cols, w.q4 ? 256 : 64);
  if (rb * cb >= ((int64_t)1 << 31)) return LORA_ERR_BAD_SHAPE;
  if (w.q4)
    hipLaunchKernelGGL(k_dequant4_t, dim3((unsigned)(rb * cb)), dim3(256), 0, st, w.codes, w.absmax,
                       w.codebook, (int)rows, (int)cols, out, ld_out, (int)cb);
  else
    hipLaunchKernelGGL(k_transpose_bf16, dim3((unsigned)(rb * cb)), dim3(256), 0, st, w.w,
                       (int)rows, (int)cols, (int64_t)cols, out, ld_out, (int)cb);
  HIP_TRY(hipGetLastError());
  return LORA_OK;
}
inline WeightView dense_view(const bf16_t *p) {
  return {false, LORA_W_DENSE, p, nullptr, AbsmaxSrc{}, nullptr, nullptr};
}

// workspace check shared by the entry points; `fast` = room for the
// weight copies
int check_ws(int op, int dtype, int wfmt, int64_t T, int64_t kd, int64_t nf, int64_t r,
             const void *ws, size_t ws_bytes, bool &fast) {
  const size_t need = lora_workspace_bytes(op | LORA_WS_MINIMAL, dtype, wfmt, T, kd, nf, r);
  if (ws_bytes < need) return LORA_ERR_WORKSPACE;
  if (need && (!ws || !aligned16(ws))) return ws ? LORA_ERR_MISALIGNED : LORA_ERR_NULL_POINTER;
  fast = ws_bytes >= lora_workspace_bytes(op, dtype, wfmt, T, kd, nf, r);
  return LORA_OK;
}

// dual pass over Z (see k_skinny_dual), then its two reductions:
//   U -> uout32 / uoutbf (k_reduce_dual_u, RSout columns, bf16 scaled by uscale)
//   V -> vout0 / vout1 (k_reduce_tn; transposed = dB layout with segment-local
//        rows, else dA layout), scaled by vscale
int skinny_dual(int RS, bool zswiglu, int64_t T, int64_t N, int64_t nsplit, int64_t ldz,
                const bf16_t *Z0, const bf16_t *Z1, const bf16_t *E, const bf16_t *G,
                const bf16_t *S0, const bf16_t *S1, const bf16_t *P0, const bf16_t *P1,
                float *part_u, float *part_v, int64_t r, int RSout, float uscale, float *uout32,
                bf16_t *uoutbf, float vscale, int transposed, bf16_t *vout0, bf16_t *vout1,
                hipStream_t st, const float *urowscale = nullptr) {
  const DualSplit sp = dual_split(T, N, nsplit, dual_slots(RS, zswiglu));
  DualArgs a{(int)T, (int)N, (int)nsplit, sp.tchunk, sp.nb0, ldz, Z0, Z1, E, G, S0, S1, P0, P1,
             (int)ldp_of(T), part_u, part_v};
  if (T > 0) {
    dim3 grid((unsigned)(sp.nb0 + sp.nb1), (unsigned)sp.ts);
#define SDU(R)                                                                              \
  case R:                                                                                   \
    if (zswiglu) hipLaunchKernelGGL((k_skinny_dual<R, R, true>), grid, dim3(256), 0, st, a); \
    else hipLaunchKernelGGL((k_skinny_dual<R, R, false>), grid, dim3(256), 0, st, a);         \
    break;
    switch (RS) {
      SDU(16) SDU(32) SDU(48) SDU(64) SDU(80) SDU(96) SDU(112) SDU(128)
      default: return LORA_ERR_UNSUPPORTED;
    }
#undef SDU
    HIP_TRY(hipGetLastError());
    ReduceUArgs ru{part_u, (int)T, RS, RSout, (int)r, sp.nb1 ? 2 : 1, sp.nb0, sp.nb1, uscale,
                   uout32, uoutbf, urowscale};
    hipLaunchKernelGGL(k_reduce_dual_u, dim3(blocks_for(T * RSout)), dim3(256), 0, st, ru);
    HIP_TRY(hipGetLastError());
  }
  ReduceTNArgs rv{part_v, T > 0 ? sp.ts : 0, RS, (int)N, (int)r, (int)nsplit, vscale, transposed,
                  vout0, vout1, 0, nullptr, 0, 0, nullptr};
  hipLaunchKernelGGL(k_reduce_tn, dim3(blocks_for((int64_t)RS * N)), dim3(256), 0, st, rv);
  HIP_TRY(hipGetLastError());
  return LORA_OK;
}

// up to three [RSout x ldp_of(T)] bf16 transposed copies, each of columns
// qoff .. qoff+nq-1 of a [T x ldin] fp32 matrix, zero elsewhere, in one launch
int pack_pt(std::initializer_list<PackJob> jobs, int64_t T, int RSout, hipStream_t st) {
  PackBatch b{};
  if (jobs.size() > 3) return LORA_ERR_UNSUPPORTED;
  for (const PackJob &j : jobs) b.j[b.n++] = j;
  b.T = (int)T; b.RSout = RSout; b.ldp = (int)ldp_of(T);
  hipLaunchKernelGGL(k_pack_pt, dim3(blocks_for((int64_t)b.n * RSout * b.ldp)), dim3(256), 0, st, b);
  HIP_TRY(hipGetLastError());
  return LORA_OK;
}

GemmArgs gemm_base() {
  GemmArgs a;
  std::memset(&a, 0, sizeof(a));
  return a;
}

void set_b(GemmArgs &a, const WeightView &w0, const WeightView &w1) {
  a.B0 = w0.w; a.B1 = w1.w;
  a.Q0 = w0.codes; a.Q1 = w1.codes;
  a.S0 = w0.absmax.absmax; a.S1 = w1.absmax.absmax;
  a.CB0 = w0.codebook; a.CB1 = w1.codebook;
  a.D0 = w0.absmax.codes; a.D1 = w1.absmax.codes;
  a.DT0 = w0.absmax.table; a.DT1 = w1.absmax.table;
  a.DS0 = w0.absmax.scale; a.DS1 = w1.absmax.scale;
  a.doff0 = w0.absmax.offset; a.doff1 = w1.absmax.offset;
}

// GEMM classes (the benchmark build's timing hook names them)
enum GemmClass {
  KC_GATEUP_FWD = 0, KC_DOWN_FWD, KC_DOWN_BWD, KC_GATEUP_BWD, KC_LINEAR_FWD, KC_LINEAR_DX,
  KC_QKV_FWD, KC_QKV_DX, KC_COUNT
};
#ifdef LORA_TIMING_HOOKS
static_assert(KC_COUNT == LORA_KC_COUNT && KC_QKV_DX == LORA_KC_QKV_DX, "class numbering");
// armed events, per host thread (liblora_timing.h)
struct TimerSlot { hipEvent_t start = nullptr, stop = nullptr; };
thread_local TimerSlot t_timer[KC_COUNT];
#endif

int run_gemm(int kc, bool nn, bool q4, int epi, const GemmArgs &a, hipStream_t st) {
  // The token operand's second source (columns >= ksplit) is addressed
  // through the first source's buffer descriptor with the constant offset
  // (A1 - A0) - ksplit elements; every caller lays the two out as column
  // ranges of one matrix, so that offset is 0.  Anything else could reach
  // past the descriptor's 2^31-byte range: refuse it.
  // (The three-source form addresses each source through its own descriptor.)
  const bool mk = a.mk_a[0] != nullptr;
  if (mk ? (nn || q4 || epi != EPI_STORE || a.mk_kb[0] != 0 || a.mk_kb[3] != a.K)
         : !(a.A1 - a.A0 == a.ksplit || (a.A1 == a.A0 && a.ksplit >= a.K)))
    return LORA_ERR_BAD_SHAPE;
#ifdef LORA_TIMING_HOOKS
  const TimerSlot ts = t_timer[kc];
  t_timer[kc] = TimerSlot{};
  if (ts.start) HIP_TRY(hipEventRecord(ts.start, st));
#endif
  hipError_t e;
  // 4-bit operands with double-quantised constants carry their 8-bit codes
  const bool dq = q4 && a.D0 != nullptr;
  if (mk)
    e = launch_gemm_nt_mk(a, st);
  else if (!nn)
    e = !q4 ? launch_gemm_nt(epi, a, st) : dq ? launch_gemm_nt_q4dq(epi, a, st)
                                              : launch_gemm_nt_q4(epi, a, st);
  else
    e = !q4 ? launch_gemm_nn(epi, a, st) : dq ? launch_gemm_nn_q4dq(epi, a, st)
                                              : launch_gemm_nn_q4(epi, a, st);
  if (e != hipSuccess) return LORA_ERR_HIP;
#ifdef LORA_TIMING_HOOKS
  if (ts.stop) HIP_TRY(hipEventRecord(ts.stop, st));
#endif
  return LORA_OK;
}

// every argument of lora_linear_bwd but the workspace
int check_lin_bwd(int dtype, int64_t T, int64_t k, int64_t n, int64_t r, const void *X,
                  const lora_weight *W, const void *A, const void *B, const void *dY, void *dX,
                  void *dA, void *dB, uint32_t flags, WeightView &wv) {
  LORA_TRY(check_dims(dtype, T, k, n, r));
  LORA_TRY(check_weight(W, dtype, k, wv));
  LORA_TRY(check_ptrs({A, B, dA, dB}));
  LORA_TRY(check_tok_ptrs(T, {X, dY}));
  if (dX && !aligned16(dX)) return LORA_ERR_MISALIGNED;
  if (flags & ~(uint32_t)LORA_FLAG_ACCUMULATE_DX) return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

// --------------------------------------------------------------- fp32 path
int gemm_f32(int64_t M, int64_t N, int64_t K, const float *A, int64_t sam, int64_t sak,
             const float *B, int64_t sbk, int64_t sbn, float *C, int64_t ldc, float alpha,
             float beta, hipStream_t st) {
  if (M == 0 || N == 0) return LORA_OK;
  F32GemmArgs a{(int)M, (int)N, (int)K, A, sam, sak, B, sbk, sbn, C, ldc, alpha, beta};
  hipLaunchKernelGGL(k_gemm_f32, dim3((unsigned)cdiv(N, 64), (unsigned)cdiv(M, 64)), dim3(256), 0,
                     st, a);
  HIP_TRY(hipGetLastError());
  return LORA_OK;
}

// Y = X W^T + s (X A^T) B^T   (fp32); H: [T x r] scratch
int lin_fwd_f32(int64_t T, int64_t k, int64_t n, int64_t r, float s, const float *X,
                const float *W, const float *A, const float *B, float *Y, float *H,
                hipStream_t st) {
  LORA_TRY(gemm_f32(T, r, k, X, k, 1, A, 1, k, H, r, 1.f, 0.f, st));
  LORA_TRY(gemm_f32(T, n, k, X, k, 1, W, 1, k, Y, n, 1.f, 0.f, st));
  LORA_TRY(gemm_f32(T, n, r, H, r, 1, B, 1, r, Y, n, s, 1.f, st));
  return LORA_OK;
}

// dX (+)= dY W + s G A;  dA = s G^T X;  dB = s dY^T H   (fp32)
int lin_bwd_f32(int64_t T, int64_t k, int64_t n, int64_t r, float s, const float *X,
                const float *W, const float *A, const float *B, const float *dY, float *dX,
                bool acc, float *dA, float *dB, float *G, float *H, hipStream_t st) {
  LORA_TRY(gemm_f32(T, r, n, dY, n, 1, B, r, 1, G, r, 1.f, 0.f, st));
  LORA_TRY(gemm_f32(T, r, k, X, k, 1, A, 1, k, H, r, 1.f, 0.f, st));
  if (dX) {
    LORA_TRY(gemm_f32(T, k, n, dY, n, 1, W, k, 1, dX, k, 1.f, acc ? 1.f : 0.f, st));
    LORA_TRY(gemm_f32(T, k, r, G, r, 1, A, k, 1, dX, k, s, 1.f, st));
  }
  LORA_TRY(gemm_f32(r, k, T, G, 1, r, X, k, 1, dA, k, s, 0.f, st));
  LORA_TRY(gemm_f32(n, r, T, dY, 1, n, H, r, 1, dB, r, s, 0.f, st));
  return LORA_OK;
}

}  // namespace

// ============================================================== public ABI
extern "C" {

int lora_abi_version(void) { return LORA_ABI_VERSION; }

#ifdef LORA_TIMING_HOOKS
int lora_debug_time_next(int which, void *start, void *stop) {
  if (which < 0 || which >= KC_COUNT) return LORA_ERR_BAD_SHAPE;
  t_timer[which] = TimerSlot{(hipEvent_t)start, (hipEvent_t)stop};
  return LORA_OK;
}
#endif

const char *lora_strerror(int status) {
  switch (status) {
    case LORA_OK: return "ok";
    case LORA_ERR_NULL_POINTER: return "null pointer argument";
    case LORA_ERR_BAD_SHAPE: return "invalid shape";
    case LORA_ERR_UNSUPPORTED: return "unsupported dtype, format or rank";
    case LORA_ERR_WORKSPACE: return "workspace too small";
    case LORA_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case LORA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t lora_workspace_bytes(int op, int dtype, int wfmt, int64_t T, int64_t kd, int64_t nf,
                            int64_t r) {
  if (op & ~(0xFF | LORA_WS_MINIMAL)) return 0;
  const bool minimal = (op & LORA_WS_MINIMAL) != 0;
  op &= 0xFF;
  if (wfmt != LORA_W_DENSE && wfmt != LORA_W_Q4 && wfmt != LORA_W_Q4_DQ) return 0;
  if (T < 0 || kd <= 0 || nf <= 0 || r <= 0 || r > LORA_MAX_RANK) return 0;
  if (dtype == LORA_F32)
    return (op == LORA_OP_RMSNORM_MLP_FWD || op == LORA_OP_RMSNORM_MLP_BWD) ? 0
                                                                            : plan_f32(op, T, kd, nf, r);
  if (dtype != LORA_BF16) return 0;
  // only 4-bit weights are copied: decoded for the forwards, decoded and
  // transposed for the backwards (dense weights are read in place: the NT
  // GEMM over a caller-kept W^T, else the NN GEMM over W as stored, which
  // costs what a per-call transposed copy would save)
  const bool fwd_copy = !minimal && wfmt != LORA_W_DENSE, bwd_copy = fwd_copy;
  switch (op) {
    case LORA_OP_LINEAR_FWD: return plan_lin_fwd(T, kd, nf, r, fwd_copy).total;
    case LORA_OP_LINEAR_BWD: return plan_lin_bwd(T, kd, nf, r, bwd_copy).total;
    case LORA_OP_MLP_FWD:
      return plan_mlp_fwd(T, kd, nf, r, fwd_copy,
                          mlp_fwd_hd_fused(r) && (wfmt == LORA_W_DENSE || fwd_copy)).total;
    case LORA_OP_MLP_BWD:
      return plan_mlp_bwd(T, kd, nf, r, bwd_copy, false,
                          mlp_bwd_hsave(r, wfmt == LORA_W_DENSE || bwd_copy)).total;
    // the folded-norm MLP takes dense weights only
    case LORA_OP_RMSNORM_MLP_FWD:
      return wfmt == LORA_W_DENSE ? plan_mlp_fwd(T, kd, nf, r, false, mlp_fwd_hd_fused(r)).total : 0;
    case LORA_OP_RMSNORM_MLP_BWD:
      return wfmt == LORA_W_DENSE
                 ? plan_mlp_bwd(T, kd, nf, r, false, true, mlp_bwd_hsave(r, true)).total
                 : 0;
  }
  return 0;
}

int lora_linear_fwd(int dtype, int64_t T, int64_t k, int64_t n, int64_t r, float alpha,
                    const void *X, const lora_weight *W, const void *A, const void *B, void *Y,
                    void *ws, size_t ws_bytes, void *stream) {
  LORA_TRY(check_dims(dtype, T, k, n, r));
  WeightView wv;
  LORA_TRY(check_weight(W, dtype, k, wv));
  LORA_TRY(check_ptrs({A, B}));
  LORA_TRY(check_tok_ptrs(T, {X, Y}));
  bool fast;
  LORA_TRY(check_ws(LORA_OP_LINEAR_FWD, dtype, W->fmt, T, k, n, r, ws, ws_bytes, fast));
  hipStream_t st = (hipStream_t)stream;
  const float s = alpha / (float)r;
  if (T == 0) return LORA_OK;
  char *w = (char *)ws;
  if (dtype == LORA_F32)
    return lin_fwd_f32(T, k, n, r, s, (const float *)X, (const float *)wv.w, (const float *)A,
                       (const float *)B, (float *)Y, (float *)w, st);

  const LinFwdPlan pl = plan_lin_fwd(T, k, n, r, fast && wv.q4);
  const int RS = rs_of(r);
  bf16_t *side_c = (bf16_t *)(w + pl.side), *epi_c = (bf16_t *)(w + pl.epi);
  // no padding: the side pass and the epilogue read A and B as they are
  const bool inplace = RS == r;
  const bf16_t *side = inplace ? (const bf16_t *)A : side_c;
  const bf16_t *epi = inplace ? (const bf16_t *)B : epi_c;
  if (fast && wv.q4) {   // decode once, then the dense GEMM
    bf16_t *wb = (bf16_t *)(w + pl.wbuf);
    LORA_TRY(decode_w(wb, wv, n, k, st));
    wv = dense_view(wb);
  }
  if (!inplace) {
    Prep prep;
    prep.side(side_c, RS, k, A, nullptr, r, k, 0);
    prep.epi(epi_c, n, RS, B, nullptr, r, n, 0);
    LORA_TRY(prep.launch(st));
  }
  GemmArgs a = gemm_base();
  a.M = (int)T; a.N = (int)n; a.K = (int)k; a.ksplit = (int)k;
  a.A0 = a.A1 = (const bf16_t *)X; a.lda = k;
  set_b(a, wv, wv); a.ldb = k;
  a.rs = RS; a.epi = epi;
  a.C = (bf16_t *)Y; a.ldc = n;
  a.tiles_m = (int)cdiv(T, BM); a.tiles_n = (int)cdiv(n, BN);
  // rank-r product s (X A^T), once per call, applied in the GEMM epilogue
  bf16_t *hbf = (bf16_t *)(w + pl.hbf);
  LORA_TRY(skinny_nt(RS, false, T, k, (const bf16_t *)X, (const bf16_t *)X, k, k, nullptr,
                     nullptr, side, (float *)(w + pl.hpart), nullptr, hbf, s, st));
  a.hglob = hbf;
  return run_gemm(KC_LINEAR_FWD, false, wv.q4, EPI_STORE, a, st);
}

int lora_linear_bwd(int dtype, int64_t T, int64_t k, int64_t n, int64_t r, float alpha,
                    const void *X, const lora_weight *W, const void *A, const void *B,
                    const void *dY, void *dX, void *dA, void *dB, uint32_t flags, void *ws,
                    size_t ws_bytes, void *stream) {
  WeightView wv;
  LORA_TRY(check_lin_bwd(dtype, T, k, n, r, X, W, A, B, dY, dX, dA, dB, flags, wv));
  bool fast;
  LORA_TRY(check_ws(LORA_OP_LINEAR_BWD, dtype, W->fmt, T, k, n, r, ws, ws_bytes, fast));
  hipStream_t st = (hipStream_t)stream;
  const float s = alpha / (float)r;
  const bool acc = (flags & LORA_FLAG_ACCUMULATE_DX) != 0;
  char *w = (char *)ws;
  if (dtype == LORA_F32) {
    float *G = (float *)w, *H = G + T * r;
    return lin_bwd_f32(T, k, n, r, s, (const float *)X, (const float *)wv.w, (const float *)A,
                       (const float *)B, (const float *)dY, (float *)dX, acc, (float *)dA,
                       (float *)dB, G, H, st);
  }
  const bool wcopy = fast && wv.q4;   // the plan holds a decoded, transposed copy
  const LinBwdPlan pl = plan_lin_bwd(T, k, n, r, wcopy);
  const int RS = rs_of(r);
  bf16_t *side_nn = (bf16_t *)(w + pl.side_nn), *epi_nn = (bf16_t *)(w + pl.epi_nn);
  bf16_t *side_nt = (bf16_t *)(w + pl.side_nt);
  float *g32 = (float *)(w + pl.g32), *h32 = (float *)(w + pl.h32);
  bf16_t *gbf = (bf16_t *)(w + pl.gbf);
  float *ntpart = (float *)(w + pl.ntpart), *tnpart = (float *)(w + pl.tnpart);
  Prep prep;
  prep.side(side_nn, RS, n, B, nullptr, r, n, 1);   // B^T padded [RS x n]
  prep.epi(epi_nn, k, RS, A, nullptr, r, k, 1);     // A^T padded [k x RS]
  prep.side(side_nt, RS, k, A, nullptr, r, k, 0);   // A padded [RS x k]
  LORA_TRY(prep.launch(st));
  const bf16_t *Xb = (const bf16_t *)X, *dYb = (const bf16_t *)dY;
  if (T > 0) {
    // G = dY B (fp32 for dA, s G in bf16 for the dX epilogue)
    LORA_TRY(skinny_nt(RS, false, T, n, dYb, dYb, n, n, nullptr, nullptr, side_nn, ntpart, g32,
                       gbf, s, st));
    if (dX) {
      GemmArgs a = gemm_base();
      a.M = (int)T; a.N = (int)k; a.K = (int)n; a.ksplit = (int)n;
      a.A0 = a.A1 = dYb; a.lda = n;
      bool nn = true, q4 = wv.q4;
      if (wcopy || wv.wt) {   // W^T [k x n] (decoded, or the caller's): NT GEMM, K-contiguous
        bf16_t *wt = wv.wt ? const_cast<bf16_t *>(wv.wt) : (bf16_t *)(w + pl.wbuf);
        if (!wv.wt) LORA_TRY(transpose_w(wt, n, wv, n, k, st));
        const WeightView tv = dense_view(wt);
        set_b(a, tv, tv); a.ldb = n;
        nn = false; q4 = false;
      } else {
        set_b(a, wv, wv); a.ldb = k;
      }
      a.rs = RS; a.epi = epi_nn;
      a.accumulate = acc; a.C = (bf16_t *)dX; a.ldc = k;
      a.hglob = gbf;
      a.tiles_m = (int)cdiv(T, BM); a.tiles_n = (int)cdiv(k, BN);
      LORA_TRY(run_gemm(KC_LINEAR_DX, nn, q4, EPI_STORE, a, st));
    }
    LORA_TRY(skinny_nt(RS, false, T, k, Xb, Xb, k, k, nullptr, nullptr, side_nt, ntpart, h32,
                       nullptr, 1.f, st));
  }
  // dA = s G^T X  [r x k];  dB = s dY^T H  [n x r]
  LORA_TRY(skinny_tn(RS, false, T, k, g32, Xb, Xb, k, k, nullptr, nullptr, tnpart, r, s, 0,
                     (bf16_t *)dA, nullptr, k, st));
  LORA_TRY(skinny_tn(RS, false, T, n, h32, dYb, dYb, n, n, nullptr, nullptr, tnpart, r, s, 1,
                     (bf16_t *)dB, nullptr, n, st));
  return LORA_OK;
}

// The allocation-free variant of lora_linear_bwd keeps its scratch memory in
// this array: one copy per GPU, held from the library's load on that device
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not the device memory: its device address is looked up once per device
// (with that device current) and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[LORA_NOALLOC_SCRATCH_BYTES];

int lora_linear_bwd_noalloc(int dtype, int64_t T, int64_t k, int64_t n, int64_t r, float alpha,
                            const void *X, const lora_weight *W, const void *A, const void *B,
                            const void *dY, void *dX, void *dA, void *dB, uint32_t flags,
                            void *stream) {
  WeightView wv;
  LORA_TRY(check_lin_bwd(dtype, T, k, n, r, X, W, A, B, dY, dX, dA, dB, flags, wv));
  // the minimal strategy's size (4-bit weights decoded inside the GEMM)
  const size_t need =
      lora_workspace_bytes(LORA_OP_LINEAR_BWD | LORA_WS_MINIMAL, dtype, W->fmt, T, k, n, r);
  if (need > (size_t)LORA_NOALLOC_SCRATCH_BYTES) return LORA_ERR_WORKSPACE;
  void *ptr = nullptr;
  if (need > 0) {
    static std::atomic<void *> dev_scratch[kMaxDevices];
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return LORA_ERR_HIP;
    ptr = dev_scratch[dev].load(std::memory_order_acquire);
    if (!ptr) {
      // the same address on every lookup for this device: a race between two
      // first calls stores it twice
      HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
      if (!ptr) return LORA_ERR_HIP;
      dev_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  return lora_linear_bwd(dtype, T, k, n, r, alpha, X, W, A, B, dY, dX, dA, dB, flags, ptr, need,
                         stream);
}

// An RMSNorm folded into the gate/up projections: the caller's gate/up
// weights are W diag(w) (lora_fold_norm_weight), the GEMMs read the raw rows
// X and scale each output row by rstd; the adapters' A become A diag(w) per
// call.  rstd is written by the forward and read by the backward.
struct NormFuse {
  const bf16_t *w;
  float eps;
  float *rstd;
  bool accumulate;   // backward: dX += the norm's input gradient
};

// every RMSNorm-specific argument; the fused path takes bf16 and dense
// weights only (a 4-bit weight cannot hold W diag(w))
static int check_norm(int dtype, int64_t T, const NormFuse &nf, const WeightView &wg,
               const WeightView &wu, const WeightView &wd) {
  if (dtype != LORA_BF16) return LORA_ERR_UNSUPPORTED;
  if (wg.q4 || wu.q4 || wd.q4) return LORA_ERR_UNSUPPORTED;
  if (!(nf.eps >= 0.f) || !std::isfinite(nf.eps)) return LORA_ERR_UNSUPPORTED;
  LORA_TRY(check_ptrs({nf.w}));
  LORA_TRY(check_tok_ptrs(T, {nf.rstd}));
  return LORA_OK;
}

static int mlp_fwd_impl(int dtype, int64_t T, int64_t d, int64_t f, int64_t r, float alpha,
                        const void *X, const lora_weight *Wg, const void *Ag, const void *Bg,
                 const lora_weight *Wu, const void *Au, const void *Bu, const lora_weight *Wd,
                 const void *Ad, const void *Bd, void *Y, void *e_saved, void *g_saved, void *ws,
                 size_t ws_bytes, void *stream, const NormFuse *nf) {
  LORA_TRY(check_dims(dtype, T, d, f, r));
  WeightView wg, wu, wd;
  LORA_TRY(check_weight(Wg, dtype, d, wg));
  LORA_TRY(check_weight(Wu, dtype, d, wu));
  LORA_TRY(check_weight(Wd, dtype, f, wd));
  if (wg.fmt != wu.fmt) return LORA_ERR_UNSUPPORTED;
  LORA_TRY(check_ptrs({Ag, Bg, Au, Bu, Ad, Bd}));
  LORA_TRY(check_tok_ptrs(T, {X, Y, e_saved, g_saved}));
  if (nf) LORA_TRY(check_norm(dtype, T, *nf, wg, wu, wd));
  bool fast;
  LORA_TRY(check_ws(nf ? LORA_OP_RMSNORM_MLP_FWD : LORA_OP_MLP_FWD, dtype, Wg->fmt, T, d, f, r, ws,
                    ws_bytes, fast));
  hipStream_t st = (hipStream_t)stream;
  const float s = alpha / (float)r;
  if (T == 0) return LORA_OK;
  char *w = (char *)ws;
  if (dtype == LORA_F32) {
    float *h = (float *)w, *H = h + T * f;
    float *e = (float *)e_saved, *g = (float *)g_saved;
    LORA_TRY(lin_fwd_f32(T, d, f, r, s, (const float *)X, (const float *)wg.w, (const float *)Ag,
                         (const float *)Bg, e, H, st));
    LORA_TRY(lin_fwd_f32(T, d, f, r, s, (const float *)X, (const float *)wu.w, (const float *)Au,
                         (const float *)Bu, g, H, st));
    hipLaunchKernelGGL(k_swiglu_f32, dim3(blocks_for(T * f)), dim3(256), 0, st, e, g, h, T * f);
    HIP_TRY(hipGetLastError());
    return lin_fwd_f32(T, f, d, r, s, h, (const float *)wd.w, (const float *)Ad,
                       (const float *)Bd, (float *)Y, H, st);
  }
  const bool wcopy = fast && wg.q4;   // the plan holds a weight buffer
  // H_d from the gate/up epilogue (eight-wave kernel: dense or decoded weights)
  const bool hdf = mlp_fwd_hd_fused(r) && (!wg.q4 || wcopy);
  // r a multiple of 16 (no padding), no folded norm and the eight-wave
  // gate/up GEMM (dense or decoded weights): every rank-r operand is an
  // adapter as it is ([Ag; Au] as two side sources, Bg / Bu read by the gate
  // and up rows, Ad, Bd), so no operand copies are made
  const bool inplace = r % 16 == 0 && !nf && (!wg.q4 || wcopy);
  const MlpFwdPlan pl = plan_mlp_fwd(T, d, f, r, wcopy, hdf);
  bf16_t *wb = (bf16_t *)(w + pl.wbuf);
  if (wcopy) {   // decode Wg, Wu once, then the dense GEMM
    LORA_TRY(decode_w(wb, wg, f, d, st));
    LORA_TRY(decode_w(wb + f * d, wu, f, d, st));
    wg = dense_view(wb);
    wu = dense_view(wb + f * d);
  }
  const int RS1 = rs_of(2 * r), RS2 = rs_of(r);
  bf16_t *h = (bf16_t *)(w + pl.h);
  bf16_t *side_gu = (bf16_t *)(w + pl.side_gu), *epi_gu = (bf16_t *)(w + pl.epi_gu);
  bf16_t *side_dc = (bf16_t *)(w + pl.side_d), *epi_dc = (bf16_t *)(w + pl.epi_d);
  // the down projection's rank-r operands: the copies, or Ad and Bd as they are
  const bf16_t *side_d = inplace ? (const bf16_t *)Ad : side_dc;
  const bf16_t *epi_d = inplace ? (const bf16_t *)Bd : epi_dc;
  bf16_t *hbf = (bf16_t *)(w + pl.hbf);
  float *hpart = (float *)(w + pl.hpart);
  if (!inplace) {
    Prep prep;
    prep.side(side_gu, RS1, d, Ag, Au, r, d, 0, nullptr, 0, nf ? nf->w : nullptr);   // [Ag; Au] (diag w)
    prep.epi(epi_gu, 2 * f, RS1, Bg, Bu, r, f, 0);
    prep.side(side_dc, RS2, f, Ad, nullptr, r, f, 0);
    prep.epi(epi_dc, d, RS2, Bd, nullptr, r, d, 0);
    LORA_TRY(prep.launch(st));
  }
  const bf16_t *Xb = (const bf16_t *)X;
  if (nf) {   // the rows' rstd only: the normalised rows are never formed
    hipLaunchKernelGGL(k_rmsnorm_fwd<false>, dim3((unsigned)cdiv(T, 4)), dim3(256), 0, st, X,
                       (const void *)nf->w, nf->eps, (int)T, (int)d, (void *)nullptr, nf->rstd);
    HIP_TRY(hipGetLastError());
  }

  // gate + up with the SwiGLU epilogue
  GemmArgs a = gemm_base();
  a.M = (int)T; a.N = (int)(2 * f); a.K = (int)d; a.ksplit = (int)d;
  a.A0 = a.A1 = Xb; a.lda = d;
  set_b(a, wg, wu); a.ldb = d;
  a.gu_f = (int)f;
  a.rs = RS1; a.epi = epi_gu;
  if (inplace) { a.epi = (const bf16_t *)Bg; a.epi_u = (const bf16_t *)Bu; }
  a.E = (bf16_t *)e_saved; a.G = (bf16_t *)g_saved; a.H = h;
  if (nf) a.rowscale = nf->rstd;
  a.tiles_m = (int)cdiv(T, BM); a.tiles_n = (int)gu_tiles_n(f);
  if (hdf) { a.fr_sd = side_d; a.fr_ud = hpart; }
  if (r % 16 == 0) a.rs_seg = (int)r;   // blockdiag(Bg, Bu): gate and up rows one block each
  // [s X Ag^T | s X Au^T], once per call
  if (inplace)
    LORA_TRY(skinny_nt(RS1, false, T, d, Xb, Xb, d, d, nullptr, nullptr, (const bf16_t *)Ag, hpart,
                       nullptr, hbf, s, st, nullptr, d, 0, (const bf16_t *)Au, (int)r));
  else
    LORA_TRY(skinny_nt(RS1, false, T, d, Xb, Xb, d, d, nullptr, nullptr, side_gu, hpart, nullptr,
                       hbf, s, st));
  a.hglob = hbf;
  LORA_TRY(run_gemm(KC_GATEUP_FWD, false, wg.q4, nf ? EPI_SWIGLU_FWD_NORM : EPI_SWIGLU_FWD, a, st));
  if (hdf) {   // s H_d in bf16: the epilogue's partials summed over the tiles in a fixed order
    const ReduceUArgs ru{hpart, (int)T, 16, RS2, (int)r, 1, (int)gu_tiles_n(f), 0, s, nullptr, hbf,
                         nullptr};
    hipLaunchKernelGGL(k_reduce_dual_u, dim3(blocks_for(T * RS2)), dim3(256), 0, st, ru);
    HIP_TRY(hipGetLastError());
  }

  // down
  if (wcopy && wd.q4) {   // reuses the buffer once the gate/up GEMM is done
    LORA_TRY(decode_w(wb, wd, d, f, st));
    wd = dense_view(wb);
  }
  GemmArgs b = gemm_base();
  b.M = (int)T; b.N = (int)d; b.K = (int)f; b.ksplit = (int)f;
  b.A0 = b.A1 = h; b.lda = f;
  set_b(b, wd, wd); b.ldb = f;
  b.rs = RS2; b.epi = epi_d;
  b.C = (bf16_t *)Y; b.ldc = d;
  b.tiles_m = (int)cdiv(T, BM); b.tiles_n = (int)cdiv(d, BN);
  // s h Ad^T, once per call, where the gate/up epilogue did not form it
  if (!hdf)
    LORA_TRY(skinny_nt(RS2, false, T, f, h, h, f, f, nullptr, nullptr, side_d, hpart, nullptr, hbf,
                       s, st));
  b.hglob = hbf;
  return run_gemm(KC_DOWN_FWD, false, wd.q4, EPI_STORE, b, st);
}

static int mlp_bwd_impl(int dtype, int64_t T, int64_t d, int64_t f, int64_t r, float alpha,
                 const void *X, const lora_weight *Wg, const void *Ag, const void *Bg,
                 const lora_weight *Wu, const void *Au, const void *Bu, const lora_weight *Wd,
                 const void *Ad, const void *Bd, const void *e_saved, const void *g_saved,
                 const void *dY, void *dX, void *dAg, void *dBg, void *dAu, void *dBu, void *dAd,
                 void *dBd, void *ws, size_t ws_bytes, void *stream, const NormFuse *nf) {
  LORA_TRY(check_dims(dtype, T, d, f, r));
  WeightView wg, wu, wd;
  LORA_TRY(check_weight(Wg, dtype, d, wg));
  LORA_TRY(check_weight(Wu, dtype, d, wu));
  LORA_TRY(check_weight(Wd, dtype, f, wd));
  if (wg.fmt != wu.fmt) return LORA_ERR_UNSUPPORTED;
  LORA_TRY(check_ptrs({Ag, Bg, Au, Bu, Ad, Bd, dAg, dBg, dAu, dBu, dAd, dBd}));
  LORA_TRY(check_tok_ptrs(T, {X, e_saved, g_saved, dY}));
  if (dX && !aligned16(dX)) return LORA_ERR_MISALIGNED;
  if (nf) LORA_TRY(check_norm(dtype, T, *nf, wg, wu, wd));
  bool fast;
  LORA_TRY(check_ws(nf ? LORA_OP_RMSNORM_MLP_BWD : LORA_OP_MLP_BWD, dtype, Wg->fmt, T, d, f, r, ws,
                    ws_bytes, fast));
  hipStream_t st = (hipStream_t)stream;
  const float s = alpha / (float)r;
  char *w = (char *)ws;

  if (dtype == LORA_F32) {
    float *h = (float *)w, *dh = h + T * f, *de = dh + T * f, *dg = de + T * f;
    float *G = dg + T * f, *H = G + T * r;
    const float *e = (const float *)e_saved, *g = (const float *)g_saved;
    if (T > 0) {
      hipLaunchKernelGGL(k_swiglu_f32, dim3(blocks_for(T * f)), dim3(256), 0, st, e, g, h, T * f);
      HIP_TRY(hipGetLastError());
    }
    LORA_TRY(lin_bwd_f32(T, f, d, r, s, h, (const float *)wd.w, (const float *)Ad,
                         (const float *)Bd, (const float *)dY, dh, false, (float *)dAd,
                         (float *)dBd, G, H, st));
    if (T > 0) {
      hipLaunchKernelGGL(k_swiglu_bwd_f32, dim3(blocks_for(T * f)), dim3(256), 0, st, e, g, dh, de,
                         dg, T * f);
      HIP_TRY(hipGetLastError());
    }
    LORA_TRY(lin_bwd_f32(T, d, f, r, s, (const float *)X, (const float *)wg.w, (const float *)Ag,
                         (const float *)Bg, de, (float *)dX, false, (float *)dAg, (float *)dBg, G,
                         H, st));
    return lin_bwd_f32(T, d, f, r, s, (const float *)X, (const float *)wu.w, (const float *)Au,
                       (const float *)Bu, dg, (float *)dX, true, (float *)dAu, (float *)dBu, G, H,
                       st);
  }

  // 4-bit gate/up weights (the format the workspace was sized for): a decoded,
  // transposed copy per dX GEMM; dense weights are read in place (NN GEMM)
  const bool wcopy = fast && wg.q4;
  const MlpBwdPlan pl =
      plan_mlp_bwd(T, d, f, r, wcopy, nf != nullptr, mlp_bwd_hsave(r, !wg.q4 || wcopy));
  // h from the down backward's epilogue: planned, and that GEMM is the
  // eight-wave kernel (a 4-bit down weight decoded in the GEMM is not)
  bf16_t *hsv = pl.hsv && !(wd.q4 && !wcopy) ? (bf16_t *)(w + pl.hsv) : nullptr;
  bf16_t *wt = (bf16_t *)(w + pl.wbuf);
  const int RS1 = rs_of(2 * r), RS2 = rs_of(r);
  bf16_t *de = (bf16_t *)(w + pl.de), *dg = (bf16_t *)(w + pl.dg);
  bf16_t *side_d_nn = (bf16_t *)(w + pl.side_d_nn), *epi_d_nn = (bf16_t *)(w + pl.epi_d_nn);
  bf16_t *side_d_nt = (bf16_t *)(w + pl.side_d_nt);
  bf16_t *epi_gu_nn = (bf16_t *)(w + pl.epi_gu_nn);
  bf16_t *side_gu_nt = (bf16_t *)(w + pl.side_gu_nt);
  bf16_t *side_g = (bf16_t *)(w + pl.side_g), *side_u = (bf16_t *)(w + pl.side_u);
  bf16_t *pt_d = (bf16_t *)(w + pl.pt_d), *pt_g = (bf16_t *)(w + pl.pt_g);
  bf16_t *pt_u = (bf16_t *)(w + pl.pt_u);
  float *part_u = (float *)(w + pl.part_u), *part_v = (float *)(w + pl.part_v);
  float *gd32 = (float *)(w + pl.gd32), *hd32 = (float *)(w + pl.hd32);
  float *ggu32 = (float *)(w + pl.ggu32), *hgu32 = (float *)(w + pl.hgu32);
  bf16_t *gdbf = (bf16_t *)(w + pl.gdbf), *ggubf = (bf16_t *)(w + pl.ggubf);
  float *ntpart = (float *)(w + pl.ntpart), *tnpart = (float *)(w + pl.tnpart);
  const bf16_t *Xb = (const bf16_t *)X, *dYb = (const bf16_t *)dY;
  const bf16_t *eb = (const bf16_t *)e_saved, *gb = (const bf16_t *)g_saved;

  Prep prep;
  prep.side(side_d_nn, RS2, d, Bd, nullptr, r, d, 1);       // Bd^T [RS2 x d]
  prep.epi(epi_d_nn, f, RS2, Ad, nullptr, r, f, 1);         // Ad^T [f x RS2]
  prep.side(side_d_nt, RS2, f, Ad, nullptr, r, f, 0);       // Ad   [RS2 x f]
  const bool dual = mlp_bwd_dual(r);
  bf16_t *side_gu_nn = (bf16_t *)(w + pl.side_gu_nn);
  if (dual) {
    prep.side(side_g, RS2, f, Bg, nullptr, r, f, 1);        // Bg^T [RS2 x f]
    prep.side(side_u, RS2, f, Bu, nullptr, r, f, 1);        // Bu^T [RS2 x f]
  } else {
    prep.side(side_gu_nn, RS1, 2 * f, Bg, Bu, r, f, 1);     // blockdiag(Bg, Bu)^T
  }
  // [Ag;Au]^T [d x RS1] and [Ag;Au] [RS1 x d], times diag(w) under a folded norm
  const bf16_t *nw = nf ? nf->w : nullptr;
  prep.epi(epi_gu_nn, d, RS1, Ag, Au, r, d, 1, nullptr, 0, nw);
  prep.side(side_gu_nt, RS1, d, Ag, Au, r, d, 0, nullptr, 0, nw);
  LORA_TRY(prep.launch(st));
  // folded norm: per-row sums of de e + dg g per 64-column block of the down
  // backward, then the coefficient of x in the norm's input gradient
  float *cpart = nf ? (float *)(w + pl.cpart) : nullptr;
  float *nkk = nf ? (float *)(w + pl.nkk) : nullptr;
  const float *rstd = nf ? nf->rstd : nullptr;

  // rank-fused: every rank-r product but dBd and dA_gu comes out of the
  // down-projection backward's epilogue (the Q4 minimal strategy's four-wave
  // GEMM has no such epilogue)
  const bool rankf = dual && mlp_bwd_rank_fused(r) && !(wd.q4 && !wcopy);
  const int64_t ftn = cdiv(f, BN), ftm = cdiv(T, BM);
  if (T > 0) {
    // 1. dh = dY Wd + s (dY Bd) Ad with the SwiGLU-derivative epilogue -> de, dg
    // G_d = dY Bd (fp32 for dAd, s G_d in bf16 for the epilogue)
    LORA_TRY(skinny_nt(RS2, false, T, d, dYb, dYb, d, d, nullptr, nullptr, side_d_nn, ntpart,
                       gd32, gdbf, s, st));
    if (rankf) {
      // the epilogue's token-contraction operands: G_d^T, and H_g^T, H_u^T
      // from H_gu = X [Ag; Au]^T
      LORA_TRY(skinny_nt(RS1, false, T, d, Xb, Xb, d, d, nullptr, nullptr, side_gu_nt, ntpart,
                         hgu32, nullptr, 1.f, st, rstd));
      LORA_TRY(pack_pt({{gd32, RS2, 0, (int)r, pt_d}, {hgu32, RS1, 0, (int)r, pt_g},
                        {hgu32, RS1, (int)r, (int)r, pt_u}}, T, RS2, st));
    }
    GemmArgs a = gemm_base();
    a.M = (int)T; a.N = (int)f; a.K = (int)d; a.ksplit = (int)d;
    a.A0 = a.A1 = dYb; a.lda = d;
    bool nn = true, q4 = wd.q4;
    if ((wcopy && wd.q4) || wd.wt) {   // Wd^T [f x d] (decoded, or the caller's)
      const bf16_t *wdt = wd.wt ? wd.wt : wt;
      if (!wd.wt) LORA_TRY(transpose_w(wt, d, wd, d, f, st));
      const WeightView tv = dense_view(wdt);
      set_b(a, tv, tv); a.ldb = d;
      nn = false; q4 = false;
    } else {
      set_b(a, wd, wd); a.ldb = f;
    }
    a.rs = RS2; a.epi = epi_d_nn;
    a.Ein = eb; a.Gin = gb; a.DE = de; a.DG = dg; a.ldd = 2 * f;
    a.H = rankf ? nullptr : hsv;
    a.hglob = gdbf;
    a.cpart = cpart;
    a.tiles_m = (int)cdiv(T, BM); a.tiles_n = (int)cdiv(f, BN);
    if (rankf) {
      a.fr_sd = side_d_nt; a.fr_sg = side_g; a.fr_su = side_u;
      a.fr_pd = pt_d; a.fr_pg = pt_g; a.fr_pu = pt_u; a.fr_ldp = (int)ldp_of(T);
      a.fr_ud = (float *)(w + pl.fu_d); a.fr_ugu = (float *)(w + pl.fu_gu);
      a.fr_vd = (float *)(w + pl.fv_d); a.fr_vgu = (float *)(w + pl.fv_gu);
    }
    LORA_TRY(run_gemm(KC_DOWN_BWD, nn, q4, rankf ? EPI_SWIGLU_BWD_RANK : EPI_SWIGLU_BWD, a, st));
    if (nf) {
      hipLaunchKernelGGL(k_norm_coef, dim3(blocks_for(T, 64)), dim3(1024), 0, st, cpart,
                         (int)(a.tiles_n * 4), (int)T, rstd, 1.0f / (float)d, nkk);
      HIP_TRY(hipGetLastError());
    }
  }
  if (rankf) {
    // the per-tile partials, reduced in a fixed order:
    //   H_d = sum over feature tiles (fp32, for dBd); dAd = s sum over token tiles;
    //   G_gu = [de Bg | dg Bu] (fp32 for dA_gu with the folded norm's rstd,
    //   s G_gu in bf16 for the dX epilogue); dBg, dBu = s sums over token tiles
    // (one launch; with T = 0 only the gradients, as zeros)
    ReduceBatch rb{};
    if (T > 0) {
      rb.u[0] = ReduceUArgs{(const float *)(w + pl.fu_d), (int)T, 16, RS2, (int)r, 1, (int)ftn, 0,
                            1.f, hd32, nullptr, nullptr};
      rb.u[1] = ReduceUArgs{(const float *)(w + pl.fu_gu), (int)T, 16, RS1, (int)r, 2, (int)ftn,
                            (int)ftn, s, ggu32, ggubf, rstd};
      rb.nu = 2;
    }
    const int tsv = T > 0 ? (int)ftm : 0;
    rb.v[0] = ReduceTNArgs{(const float *)(w + pl.fv_d), tsv, 16, (int)f, (int)r, (int)f, s, 0,
                           (bf16_t *)dAd, nullptr, 0, nullptr, 0, 0, nullptr};
    rb.v[1] = ReduceTNArgs{(const float *)(w + pl.fv_gu), tsv, 16, (int)(2 * f), (int)r, (int)f, s,
                           1, (bf16_t *)dBg, (bf16_t *)dBu, 0, nullptr, 0, 0, nullptr};
    rb.nv = 2;
    const int64_t cnt[4] = {T * RS2, T * RS1, (int64_t)16 * f, (int64_t)16 * 2 * f};
    int64_t nblk = 0;
    for (int j = 0, c = rb.nu ? 0 : 2; c < 4; ++j, ++c) {
      rb.start[j] = nblk;
      nblk += blocks_for(cnt[c]);
    }
    rb.start[rb.nu + rb.nv] = nblk;
    hipLaunchKernelGGL(k_reduce_batch, dim3((unsigned)nblk), dim3(256), 0, st, rb);
    HIP_TRY(hipGetLastError());
  }
  // 2. one pass over h = silu(e) g (recomputed): H_d = h Ad^T (fp32, for dBd)
  //    and dAd = s G_d^T h
  if (rankf) {
    // formed by the down backward's epilogue
  } else if (dual) {
    if (T > 0) LORA_TRY(pack_pt({{gd32, RS2, 0, (int)r, pt_d}}, T, RS2, st));   // G_d^T bf16
    LORA_TRY(skinny_dual(RS2, true, T, f, f, f, nullptr, nullptr, eb, gb, side_d_nt, nullptr,
                         pt_d, nullptr, part_u, part_v, r, RS2, 1.f, hd32, nullptr, s, 0,
                         (bf16_t *)dAd, nullptr, st));
  } else if (hsv) {   // over h as the down backward's epilogue stored it
    LORA_TRY(skinny_nt(RS2, false, T, f, hsv, hsv, f, f, nullptr, nullptr, side_d_nt, ntpart, hd32,
                       nullptr, 1.f, st));
    LORA_TRY(skinny_tn(RS2, false, T, f, gd32, hsv, hsv, f, f, nullptr, nullptr, tnpart, r, s, 0,
                       (bf16_t *)dAd, nullptr, f, st));
  } else {
    LORA_TRY(skinny_nt(RS2, true, T, f, nullptr, nullptr, f, f, eb, gb, side_d_nt, ntpart, hd32,
                       nullptr, 1.f, st));
    LORA_TRY(skinny_tn(RS2, true, T, f, gd32, nullptr, nullptr, f, f, eb, gb, tnpart, r, s, 0,
                       (bf16_t *)dAd, nullptr, f, st));
  }
  // 3. dBd = s dY^T H_d
  LORA_TRY(skinny_tn(RS2, false, T, d, hd32, dYb, dYb, d, d, nullptr, nullptr, tnpart, r, s, 1,
                     (bf16_t *)dBd, nullptr, d, st));
  if (T > 0 && !rankf) {
    // 4. H_gu = X [Ag; Au]^T (fp32), its two halves transposed to bf16
    LORA_TRY(skinny_nt(RS1, false, T, d, Xb, Xb, d, d, nullptr, nullptr, side_gu_nt, ntpart, hgu32,
                       nullptr, 1.f, st, rstd));
    if (dual) {
      LORA_TRY(pack_pt({{hgu32, RS1, 0, (int)r, pt_g}, {hgu32, RS1, (int)r, (int)r, pt_u}}, T,
                       RS2, st));
    }
  }
  // 5. G_gu = [de Bg | dg Bu] (fp32 for dA_gu, s G_gu in bf16 for the dX
  //    epilogue) and dBg = s de^T H_g, dBu = s dg^T H_u: one pass over [de | dg]
  if (rankf) {
    // formed by the down backward's epilogue
  } else if (dual) {
    LORA_TRY(skinny_dual(RS2, false, T, 2 * f, f, 2 * f, de, dg, nullptr, nullptr, side_g, side_u,
                         pt_g, pt_u, part_u, part_v, r, RS1, s, ggu32, ggubf, s, 1, (bf16_t *)dBg,
                         (bf16_t *)dBu, st, rstd));
  } else if (mlp_bwd_gu_segmented(r)) {
    // block-diagonal in the rank: de with Bg and H_g, dg with Bu and H_u,
    // each an r-wide pass over its half of [de | dg]
    const bf16_t *zs[2] = {de, dg};
    bf16_t *dbs[2] = {(bf16_t *)dBg, (bf16_t *)dBu};
    for (int j = 0; j < 2; ++j) {
      if (T > 0)
        LORA_TRY(skinny_nt((int)r, false, T, f, zs[j], zs[j], f, 2 * f, nullptr, nullptr,
                           side_gu_nn + (int64_t)j * r * 2 * f + j * f, ntpart, ggu32 + j * r,
                           ggubf + j * r, s, st, rstd, 2 * f, RS1));
      LORA_TRY(skinny_tn((int)r, false, T, f, hgu32 + j * r, zs[j], zs[j], f, 2 * f, nullptr, nullptr,
                         tnpart, r, s, 1, dbs[j], nullptr, f, st, nullptr, 0, nullptr, RS1));
    }
  } else {
    if (T > 0)
      LORA_TRY(skinny_nt(RS1, false, T, 2 * f, de, dg, f, 2 * f, nullptr, nullptr, side_gu_nn, ntpart,
                         ggu32, ggubf, s, st, rstd));
    LORA_TRY(skinny_tn(RS1, false, T, 2 * f, hgu32, de, dg, f, 2 * f, nullptr, nullptr, tnpart, r, s,
                       1, (bf16_t *)dBg, (bf16_t *)dBu, f, st));
  }
  if (T > 0 && dX) {
    // 6. dX = de Wg + dg Wu + s [de Bg | dg Bu] [Ag; Au]
    GemmArgs b = gemm_base();
    b.M = (int)T; b.N = (int)d; b.K = (int)(2 * f); b.ksplit = (int)f;
    b.A0 = de; b.A1 = dg; b.lda = 2 * f;
    bool nn = true, q4 = wg.q4;
    if (wcopy) {   // decoded [Wg^T | Wu^T] [d x 2f], over Wd^T (its GEMM is done)
      LORA_TRY(transpose_w(wt, 2 * f, wg, f, d, st));
      LORA_TRY(transpose_w(wt + f, 2 * f, wu, f, d, st));
      const WeightView tv = dense_view(wt);
      set_b(b, tv, tv); b.ldb = 2 * f;
      nn = false; q4 = false;
    } else if (wg.wt && wu.wt && f % 64 == 0) {
      // the caller's Wg^T, Wu^T [d x f]: the K halves of one NT product
      const WeightView tv = dense_view(wg.wt);
      set_b(b, tv, tv); b.ldb = f;
      b.Bk1 = wu.wt; b.kbsplit = (int)f;
      nn = false;
    } else {
      set_b(b, wg, wu); b.ldb = d;
    }
    b.rs = RS1; b.epi = epi_gu_nn;
    b.C = (bf16_t *)dX; b.ldc = d;
    b.hglob = ggubf;
    if (nf) {   // dX = rstd gn - kk x (+ the residual stream's gradient)
      b.nrm_x = Xb; b.nrm_rs = rstd; b.nrm_kk = nkk;
      b.accumulate = nf->accumulate;
    }
    b.tiles_m = (int)cdiv(T, BM); b.tiles_n = (int)cdiv(d, BN);
    LORA_TRY(run_gemm(KC_GATEUP_BWD, nn, q4, nf ? EPI_STORE_NORM : EPI_STORE, b, st));
  }
  // 7. [dAg; dAu] = s G_gu^T X  (folded norm: G_gu rows scaled by rstd, the
  //    result's columns by w, so X stands in for the normalised rows)
  LORA_TRY(skinny_tn(RS1, false, T, d, ggu32, Xb, Xb, d, d, nullptr, nullptr, tnpart, r, s, 0,
                     (bf16_t *)dAg, (bf16_t *)dAu, d, st, nullptr, 0, nw));
  return LORA_OK;
}

int lora_swiglu_mlp_fwd(int dtype, int64_t T, int64_t d, int64_t f, int64_t r, float alpha,
                        const void *X, const lora_weight *Wg, const void *Ag, const void *Bg,
                        const lora_weight *Wu, const void *Au, const void *Bu,
                        const lora_weight *Wd, const void *Ad, const void *Bd, void *Y,
                        void *e_saved, void *g_saved, void *ws, size_t ws_bytes, void *stream) {
  return mlp_fwd_impl(dtype, T, d, f, r, alpha, X, Wg, Ag, Bg, Wu, Au, Bu, Wd, Ad, Bd, Y, e_saved,
                      g_saved, ws, ws_bytes, stream, nullptr);
}

int lora_swiglu_mlp_bwd(int dtype, int64_t T, int64_t d, int64_t f, int64_t r, float alpha,
                        const void *X, const lora_weight *Wg, const void *Ag, const void *Bg,
                        const lora_weight *Wu, const void *Au, const void *Bu,
                        const lora_weight *Wd, const void *Ad, const void *Bd,
                        const void *e_saved, const void *g_saved, const void *dY, void *dX,
                        void *dAg, void *dBg, void *dAu, void *dBu, void *dAd, void *dBd,
                        void *ws, size_t ws_bytes, void *stream) {
  return mlp_bwd_impl(dtype, T, d, f, r, alpha, X, Wg, Ag, Bg, Wu, Au, Bu, Wd, Ad, Bd, e_saved,
                      g_saved, dY, dX, dAg, dBg, dAu, dBu, dAd, dBd, ws, ws_bytes, stream, nullptr);
}

int lora_rmsnorm_swiglu_mlp_fwd(int dtype, int64_t T, int64_t d, int64_t f, int64_t r, float alpha,
                                float eps, const void *X, const void *norm_w,
                                const lora_weight *Wg, const void *Ag, const void *Bg,
                                const lora_weight *Wu, const void *Au, const void *Bu,
                                const lora_weight *Wd, const void *Ad, const void *Bd, void *Y,
                                void *e_saved, void *g_saved, float *rstd, void *ws,
                                size_t ws_bytes, void *stream) {
  const NormFuse nf{(const bf16_t *)norm_w, eps, rstd, false};
  return mlp_fwd_impl(dtype, T, d, f, r, alpha, X, Wg, Ag, Bg, Wu, Au, Bu, Wd, Ad, Bd, Y, e_saved,
                      g_saved, ws, ws_bytes, stream, &nf);
}

int lora_rmsnorm_swiglu_mlp_bwd(int dtype, int64_t T, int64_t d, int64_t f, int64_t r, float alpha,
                                const void *X, const void *norm_w, const float *rstd,
                                const lora_weight *Wg, const void *Ag, const void *Bg,
                                const lora_weight *Wu, const void *Au, const void *Bu,
                                const lora_weight *Wd, const void *Ad, const void *Bd,
                                const void *e_saved, const void *g_saved, const void *dY, void *dX,
                                void *dAg, void *dBg, void *dAu, void *dBu, void *dAd, void *dBd,
                                uint32_t flags, void *ws, size_t ws_bytes, void *stream) {
  if (flags & ~(uint32_t)LORA_FLAG_ACCUMULATE_DX) return LORA_ERR_UNSUPPORTED;
  const NormFuse nf{(const bf16_t *)norm_w, 0.f, const_cast<float *>(rstd),
                    (flags & LORA_FLAG_ACCUMULATE_DX) != 0};
  return mlp_bwd_impl(dtype, T, d, f, r, alpha, X, Wg, Ag, Bg, Wu, Au, Bu, Wd, Ad, Bd, e_saved,
                      g_saved, dY, dX, dAg, dBg, dAu, dBu, dAd, dBd, ws, ws_bytes, stream, &nf);
}

int lora_fold_norm_weight(int dtype, int64_t n, int64_t k, const void *W, const void *norm_w,
                          void *out, void *stream) {
  if (dtype != LORA_BF16) return LORA_ERR_UNSUPPORTED;
  if (n <= 0 || k <= 0 || n > kMaxFeatures || k > kMaxFeatures || (k % 8)) return LORA_ERR_BAD_SHAPE;
  LORA_TRY(check_ptrs({W, norm_w, out}));
  if (n * k == 0) return LORA_OK;
  hipLaunchKernelGGL(k_fold_colscale, dim3(blocks_for(n * k / 8)), dim3(256), 0,
                     (hipStream_t)stream, (const bf16_t *)W, (const bf16_t *)norm_w, n, k,
                     (bf16_t *)out);
  HIP_TRY(hipGetLastError());
  return LORA_OK;
}

size_t lora_qkv_workspace_bytes(int op, int dtype, int wfmt, int64_t T, int64_t k, int64_t nq,
                                int64_t nkv, int64_t r) {
  if (op & ~(0xFF | LORA_WS_MINIMAL)) return 0;
  const bool minimal = (op & LORA_WS_MINIMAL) != 0;
  const int base = op & 0xFF;
  if (base == LORA_OP_RMSNORM_QKV_FWD || base == LORA_OP_RMSNORM_QKV_BWD) {
    // one strategy (bf16, dense weights, the stacked GEMM's shapes)
    if (dtype != LORA_BF16 || wfmt != LORA_W_DENSE || !qkv_shapes_ok(k, nq, nkv, r)) return 0;
    if (T < 0 || T > ((int64_t)1 << 30)) return 0;
    return base == LORA_OP_RMSNORM_QKV_FWD ? plan_qkv_fwd(T, k, nq, nkv, r, false).total
                                           : plan_qkv_bwd(T, k, nq, nkv, r, true).total;
  }
  if (base != LORA_OP_QKV_FWD && base != LORA_OP_QKV_BWD) return 0;
  if (wfmt != LORA_W_DENSE && wfmt != LORA_W_Q4 && wfmt != LORA_W_Q4_DQ) return 0;
  if (T < 0 || k <= 0 || nq <= 0 || nkv <= 0 || r <= 0 || r > LORA_MAX_RANK) return 0;
  const int lop = base == LORA_OP_QKV_FWD ? LORA_OP_LINEAR_FWD : LORA_OP_LINEAR_BWD;
  const int mflag = minimal ? LORA_WS_MINIMAL : 0;
  // the per-projection calls (used for shapes and strategies the fused
  // kernels do not take) share the workspace
  size_t need = std::max(lora_workspace_bytes(lop | mflag, dtype, wfmt, T, k, nq, r),
                         lora_workspace_bytes(lop | mflag, dtype, wfmt, T, k, nkv, r));
  if (need == 0 && dtype == LORA_BF16) return 0;
  if (dtype == LORA_BF16 && qkv_rank_ok(r)) {
    if (base == LORA_OP_QKV_FWD)
      need = std::max(need,
                      plan_qkv_fwd(T, k, nq, nkv, r, !minimal && wfmt != LORA_W_DENSE).total);
    else if (!minimal)
      need = std::max(need, plan_qkv_bwd(T, k, nq, nkv, r).total);
  }
  return need;
}

// The stacked q/k/v forward (bf16, nq and nkv multiples of the tile width,
// 3r <= 256): one rank-3r pass over X and one GEMM over [Wq; Wk; Wv] whose
// store epilogue writes Q, K, V.  With a folded norm the GEMM reads the raw
// rows and scales each output row by rstd.
static int qkv_fwd_fused(int64_t T, int64_t k, int64_t nq, int64_t nkv, int64_t r, float alpha,
                         const void *X, WeightView wq, WeightView wk, WeightView wv,
                         const void *Aq, const void *Bq, const void *Ak, const void *Bk,
                         const void *Av, const void *Bv, void *Q, void *K, void *V, void *ws,
                         hipStream_t st, const NormFuse *nf) {
  const int64_t N = nq + 2 * nkv;
  const int RS3 = rs_of(3 * r);
  const float s = alpha / (float)r;
  char *w = (char *)ws;
  const QkvFwdPlan pl = plan_qkv_fwd(T, k, nq, nkv, r, wq.q4);
  bf16_t *side = (bf16_t *)(w + pl.side), *epi = (bf16_t *)(w + pl.epi);
  bf16_t *hbf = (bf16_t *)(w + pl.hbf);
  if (wq.q4) {   // decode the three weights once, stacked [Wq; Wk; Wv]
    bf16_t *wb = (bf16_t *)(w + pl.wbuf);
    LORA_TRY(decode_w(wb, wq, nq, k, st));
    LORA_TRY(decode_w(wb + nq * k, wk, nkv, k, st));
    LORA_TRY(decode_w(wb + (nq + nkv) * k, wv, nkv, k, st));
    wq = dense_view(wb);
    wk = dense_view(wb + nq * k);
    wv = dense_view(wb + (nq + nkv) * k);
  }
  Prep prep;
  // [Aq; Ak; Av], times diag(w) under a folded norm
  prep.side(side, RS3, k, Aq, Ak, r, k, 0, Av, k, nf ? nf->w : nullptr);
  prep.epi(epi, N, RS3, Bq, Bk, r, nq, 0, Bv, nq + nkv);            // blockdiag(Bq, Bk, Bv)
  LORA_TRY(prep.launch(st));
  const bf16_t *Xb = (const bf16_t *)X;
  if (nf) {   // the rows' rstd only: the normalised rows are never formed
    hipLaunchKernelGGL(k_rmsnorm_fwd<false>, dim3((unsigned)cdiv(T, 4)), dim3(256), 0, st, X,
                       (const void *)nf->w, nf->eps, (int)T, (int)k, (void *)nullptr, nf->rstd);
    HIP_TRY(hipGetLastError());
  }
  LORA_TRY(skinny_nt(RS3, false, T, k, Xb, Xb, k, k, nullptr, nullptr, side,
                     (float *)(w + pl.hpart), nullptr, hbf, s, st));
  GemmArgs a = gemm_base();
  a.M = (int)T; a.N = (int)N; a.K = (int)k; a.ksplit = (int)k;
  a.A0 = a.A1 = Xb; a.lda = k;
  a.B0 = wq.w; a.B1 = wk.w; a.B2 = wv.w; a.ldb = k;
  a.nseg1 = (int)nq; a.nseg2 = (int)(nq + nkv);
  a.rs = RS3; a.epi = epi; a.hglob = hbf;
  if (r % 16 == 0) a.rs_seg = (int)r;   // blockdiag(Bq, Bk, Bv): one block per tile
  if (nf) a.rowscale = nf->rstd;
  a.C = (bf16_t *)Q; a.ldc = nq;
  a.C1 = (bf16_t *)K; a.ldc1 = nkv;
  a.C2 = (bf16_t *)V; a.ldc2 = nkv;
  a.tiles_m = (int)cdiv(T, BM); a.tiles_n = (int)(N / BN);
  return run_gemm(KC_QKV_FWD, false, false, nf ? EPI_STORE_NORM : EPI_STORE, a, st);
}

int lora_qkv_fwd(int dtype, int64_t T, int64_t k, int64_t nq, int64_t nkv, int64_t r,
                 float alpha, const void *X, const lora_weight *Wq, const void *Aq,
                 const void *Bq, const lora_weight *Wk, const void *Ak, const void *Bk,
                 const lora_weight *Wv, const void *Av, const void *Bv, void *Q, void *K,
                 void *V, void *ws, size_t ws_bytes, void *stream) {
  LORA_TRY(check_dims(dtype, T, k, nq, r));
  LORA_TRY(check_dims(dtype, T, k, nkv, r));
  WeightView wq, wk, wv;
  LORA_TRY(check_weight(Wq, dtype, k, wq));
  LORA_TRY(check_weight(Wk, dtype, k, wk));
  LORA_TRY(check_weight(Wv, dtype, k, wv));
  if (wq.fmt != wk.fmt || wq.fmt != wv.fmt) return LORA_ERR_UNSUPPORTED;
  LORA_TRY(check_ptrs({Aq, Bq, Ak, Bk, Av, Bv}));
  LORA_TRY(check_tok_ptrs(T, {X, Q, K, V}));
  const size_t need = lora_qkv_workspace_bytes(LORA_OP_QKV_FWD | LORA_WS_MINIMAL, dtype, Wq->fmt,
                                               T, k, nq, nkv, r);
  if (ws_bytes < need) return LORA_ERR_WORKSPACE;
  if (need && (!ws || !aligned16(ws))) return ws ? LORA_ERR_MISALIGNED : LORA_ERR_NULL_POINTER;
  const bool fast =
      ws_bytes >= lora_qkv_workspace_bytes(LORA_OP_QKV_FWD, dtype, Wq->fmt, T, k, nq, nkv, r);
  if (T == 0) return LORA_OK;
  hipStream_t st = (hipStream_t)stream;
  const bool fused = dtype == LORA_BF16 && qkv_rank_ok(r) && nq % BN == 0 && nkv % BN == 0 &&
                     (!wq.q4 || fast);
  if (!fused) {   // one LoRA linear per projection, same kernels
    LORA_TRY(lora_linear_fwd(dtype, T, k, nq, r, alpha, X, Wq, Aq, Bq, Q, ws, ws_bytes, stream));
    LORA_TRY(lora_linear_fwd(dtype, T, k, nkv, r, alpha, X, Wk, Ak, Bk, K, ws, ws_bytes, stream));
    return lora_linear_fwd(dtype, T, k, nkv, r, alpha, X, Wv, Av, Bv, V, ws, ws_bytes, stream);
  }
  return qkv_fwd_fused(T, k, nq, nkv, r, alpha, X, wq, wk, wv, Aq, Bq, Ak, Bk, Av, Bv, Q, K, V, ws,
                       st, nullptr);
}

// The stacked q/k/v backward (bf16, fast workspace, 3r <= 256): [dQ | dK | dV]
// packed once, one rank-3r pass for G, one dX GEMM with K = nq + 2 nkv over
// the transposed stacked weights, one pass for H and the two adapter-gradient
// passes.  With a folded norm the adapters' A become A diag(w), the rank-r
// products carry rstd, and dX is the raw rows' gradient.
static int qkv_bwd_fused(int64_t T, int64_t k, int64_t nq, int64_t nkv, int64_t r, float alpha,
                         const void *X, WeightView wq, WeightView wk, WeightView wv,
                         const void *Aq, const void *Bq, const void *Ak, const void *Bk,
                         const void *Av, const void *Bv, const void *dQ, const void *dK,
                         const void *dV, void *dX, void *dAq, void *dBq, void *dAk, void *dBk,
                         void *dAv, void *dBv, bool acc, void *ws, hipStream_t st,
                         const NormFuse *nf) {
  const int64_t N = nq + 2 * nkv;
  const int RS3 = rs_of(3 * r);
  const float s = alpha / (float)r;
  char *w = (char *)ws;
  const QkvBwdPlan pl = plan_qkv_bwd(T, k, nq, nkv, r, nf != nullptr);
  const bf16_t *nw = nf ? nf->w : nullptr;
  const float *rstd = nf ? nf->rstd : nullptr;
  bf16_t *dyc = (bf16_t *)(w + pl.dyc), *wt = (bf16_t *)(w + pl.wbuf);
  bf16_t *side_nn = (bf16_t *)(w + pl.side_nn), *epi_nn = (bf16_t *)(w + pl.epi_nn);
  bf16_t *side_nt = (bf16_t *)(w + pl.side_nt), *gbf = (bf16_t *)(w + pl.gbf);
  float *g32 = (float *)(w + pl.g32), *h32 = (float *)(w + pl.h32);
  float *ntpart = (float *)(w + pl.ntpart), *tnpart = (float *)(w + pl.tnpart);
  const bf16_t *Xb = (const bf16_t *)X;
  // the three gradients as they are, their widths and first columns in [dQ | dK | dV]
  const bool seg = qkv_bwd_segmented(r);
  const bf16_t *sd[3] = {(const bf16_t *)dQ, (const bf16_t *)dK, (const bf16_t *)dV};
  const int64_t sn[3] = {nq, nkv, nkv}, sc[3] = {0, nq, nq + nkv};
  Prep prep;
  prep.side(side_nn, RS3, N, Bq, Bk, r, nq, 1, Bv, nq + nkv);       // blockdiag(Bq,Bk,Bv)^T
  // [Aq; Ak; Av]^T and [Aq; Ak; Av], times diag(w) under a folded norm
  prep.epi(epi_nn, k, RS3, Aq, Ak, r, k, 1, Av, k, nw);
  prep.side(side_nt, RS3, k, Aq, Ak, r, k, 0, Av, k, nw);
  LORA_TRY(prep.launch(st));
  if (T > 0) {
    // the dX GEMM reads dQ, dK, dV and the three W^T as three K sources when
    // the projection widths are multiples of the K step
    const bool mk = nq % 64 == 0 && nkv % 64 == 0;
    // [dQ | dK | dV] as one [T x N] operand (for the dX GEMM over one K source,
    // and for the rank passes unless they run block by block)
    if ((dX && !mk) || !seg) {
      hipLaunchKernelGGL(k_concat3, dim3(blocks_for(T * (N / 8))), dim3(256), 0, st,
                         (const bf16_t *)dQ, (const bf16_t *)dK, (const bf16_t *)dV, (int)nq,
                         (int)nkv, (int)nkv, T, dyc);
      HIP_TRY(hipGetLastError());
    }
    // G = [dQ Bq | dK Bk | dV Bv] (fp32 for dA, rows times rstd under a
    // folded norm; s G in bf16 for the dX epilogue)
    if (seg) {   // block by block: the rows of blockdiag(Bq, Bk, Bv)^T that are not zero
      for (int j = 0; j < 3; ++j)
        LORA_TRY(skinny_nt((int)r, false, T, sn[j], sd[j], sd[j], sn[j], sn[j], nullptr, nullptr,
                           side_nn + (int64_t)j * r * N + sc[j], ntpart, g32 + j * r, gbf + j * r, s,
                           st, rstd, N, RS3));
    } else {
      LORA_TRY(skinny_nt(RS3, false, T, N, dyc, dyc, N, N, nullptr, nullptr, side_nn, ntpart, g32,
                         gbf, s, st, rstd));
    }
    if (dX) {
      // dX (+)= [dQ | dK | dV] [Wq; Wk; Wv] + s G [Aq; Ak; Av]: one GEMM, K = N,
      // over the three W^T (the caller's, else transposed here, stacked)
      const bool kept = mk && wq.wt && wk.wt && wv.wt;
      if (!kept) {
        LORA_TRY(transpose_w(wt, N, wq, nq, k, st));
        LORA_TRY(transpose_w(wt + nq, N, wk, nkv, k, st));
        LORA_TRY(transpose_w(wt + nq + nkv, N, wv, nkv, k, st));
      }
      GemmArgs a = gemm_base();
      a.M = (int)T; a.N = (int)k; a.K = (int)N; a.ksplit = (int)N;
      if (mk) {
        const bf16_t *gs[3] = {(const bf16_t *)dQ, (const bf16_t *)dK, (const bf16_t *)dV};
        const bf16_t *ws3[3] = {wq.wt, wk.wt, wv.wt};
        for (int j = 0; j < 3; ++j) {
          a.mk_a[j] = gs[j];
          a.mk_lda[j] = sn[j];
          a.mk_b[j] = kept ? ws3[j] : wt + sc[j];
          a.mk_ldb[j] = kept ? sn[j] : N;
          a.mk_kb[j] = (int)sc[j];
        }
        a.mk_kb[3] = (int)N;
      } else {
        a.A0 = a.A1 = dyc; a.lda = N;
        const WeightView tv = dense_view(wt);
        set_b(a, tv, tv); a.ldb = N;
      }
      a.rs = RS3; a.epi = epi_nn; a.hglob = gbf;
      // folded norm: the GEMM gives gn, the gradient with respect to X rstd
      bf16_t *gn = nf ? (bf16_t *)(w + pl.gn) : (bf16_t *)dX;
      a.accumulate = !nf && acc; a.C = gn; a.ldc = k;
      a.tiles_m = (int)cdiv(T, BM); a.tiles_n = (int)cdiv(k, BN);
      LORA_TRY(run_gemm(KC_QKV_DX, false, false, EPI_STORE, a, st));
      if (nf) {   // dX (+)= rstd gn - rstd^3 X (sum_j gn_j X_j) / k (unit norm weight)
        hipLaunchKernelGGL(k_rmsnorm_bwd<false>, dim3((unsigned)cdiv(T, 4)), dim3(256), 0, st, X,
                           (const void *)nullptr, rstd, (const void *)gn, (int)T, (int)k, dX,
                           acc ? 1 : 0);
        HIP_TRY(hipGetLastError());
      }
    }
    // H = X [Aq; Ak; Av]^T (folded norm: rstd X [Aq; Ak; Av]^T diag(w), the
    // normalised rows' product)
    LORA_TRY(skinny_nt(RS3, false, T, k, Xb, Xb, k, k, nullptr, nullptr, side_nt, ntpart, h32,
                       nullptr, 1.f, st, rstd));
  }
  // [dAq; dAk; dAv] = s G^T X ;  dBq = s dQ^T H_q, dBk = s dK^T H_k, dBv = s dV^T H_v
  //   (folded norm: G rows scaled by rstd, the result's columns by w)
  LORA_TRY(skinny_tn(RS3, false, T, k, g32, Xb, Xb, k, k, nullptr, nullptr, tnpart, r, s, 0,
                     (bf16_t *)dAq, (bf16_t *)dAk, k, st, (bf16_t *)dAv, 0, nw));
  if (seg) {   // dB_j = s dY_j^T H_j, each over its own gradient and rank block of H
    bf16_t *dBs[3] = {(bf16_t *)dBq, (bf16_t *)dBk, (bf16_t *)dBv};
    for (int j = 0; j < 3; ++j)
      LORA_TRY(skinny_tn((int)r, false, T, sn[j], h32 + j * r, sd[j], sd[j], sn[j], sn[j], nullptr,
                         nullptr, tnpart, r, s, 1, dBs[j], nullptr, sn[j], st, nullptr, 0, nullptr,
                         RS3));
  } else {
    LORA_TRY(skinny_tn(RS3, false, T, N, h32, dyc, dyc, N, N, nullptr, nullptr, tnpart, r, s, 1,
                       (bf16_t *)dBq, (bf16_t *)dBk, nq, st, (bf16_t *)dBv, nq + nkv));
  }
  return LORA_OK;
}

int lora_qkv_bwd(int dtype, int64_t T, int64_t k, int64_t nq, int64_t nkv, int64_t r,
                 float alpha, const void *X, const lora_weight *Wq, const void *Aq,
                 const void *Bq, const lora_weight *Wk, const void *Ak, const void *Bk,
                 const lora_weight *Wv, const void *Av, const void *Bv, const void *dQ,
                 const void *dK, const void *dV, void *dX, void *dAq, void *dBq, void *dAk,
                 void *dBk, void *dAv, void *dBv, uint32_t flags, void *ws, size_t ws_bytes,
                 void *stream) {
  LORA_TRY(check_dims(dtype, T, k, nq, r));
  LORA_TRY(check_dims(dtype, T, k, nkv, r));
  WeightView wq, wk, wv;
  LORA_TRY(check_weight(Wq, dtype, k, wq));
  LORA_TRY(check_weight(Wk, dtype, k, wk));
  LORA_TRY(check_weight(Wv, dtype, k, wv));
  if (wq.fmt != wk.fmt || wq.fmt != wv.fmt) return LORA_ERR_UNSUPPORTED;
  LORA_TRY(check_ptrs({Aq, Bq, Ak, Bk, Av, Bv, dAq, dBq, dAk, dBk, dAv, dBv}));
  LORA_TRY(check_tok_ptrs(T, {X, dQ, dK, dV}));
  if (dX && !aligned16(dX)) return LORA_ERR_MISALIGNED;
  if (flags & ~(uint32_t)LORA_FLAG_ACCUMULATE_DX) return LORA_ERR_UNSUPPORTED;
  const size_t need = lora_qkv_workspace_bytes(LORA_OP_QKV_BWD | LORA_WS_MINIMAL, dtype, Wq->fmt,
                                               T, k, nq, nkv, r);
  if (ws_bytes < need) return LORA_ERR_WORKSPACE;
  if (need && (!ws || !aligned16(ws))) return ws ? LORA_ERR_MISALIGNED : LORA_ERR_NULL_POINTER;
  const bool fast =
      ws_bytes >= lora_qkv_workspace_bytes(LORA_OP_QKV_BWD, dtype, Wq->fmt, T, k, nq, nkv, r);
  hipStream_t st = (hipStream_t)stream;
  const bool fused = dtype == LORA_BF16 && qkv_rank_ok(r) && fast;
  if (!fused) {   // one LoRA linear per projection; their dX contributions accumulate
    LORA_TRY(lora_linear_bwd(dtype, T, k, nq, r, alpha, X, Wq, Aq, Bq, dQ, dX, dAq, dBq, flags,
                             ws, ws_bytes, stream));
    LORA_TRY(lora_linear_bwd(dtype, T, k, nkv, r, alpha, X, Wk, Ak, Bk, dK, dX, dAk, dBk,
                             LORA_FLAG_ACCUMULATE_DX, ws, ws_bytes, stream));
    return lora_linear_bwd(dtype, T, k, nkv, r, alpha, X, Wv, Av, Bv, dV, dX, dAv, dBv,
                           LORA_FLAG_ACCUMULATE_DX, ws, ws_bytes, stream);
  }
  return qkv_bwd_fused(T, k, nq, nkv, r, alpha, X, wq, wk, wv, Aq, Bq, Ak, Bk, Av, Bv, dQ, dK, dV,
                       dX, dAq, dBq, dAk, dBk, dAv, dBv, (flags & LORA_FLAG_ACCUMULATE_DX) != 0,
                       ws, st, nullptr);
}

// checks shared by the norm-fused q/k/v entry points: bf16, dense weights and
// the shapes of the stacked GEMM (the projections one by one cannot take a
// folded norm: their per-call rank products carry no rstd)
static int check_qkv_norm(int dtype, int64_t T, int64_t k, int64_t nq, int64_t nkv, int64_t r,
                          const lora_weight *Wq, const lora_weight *Wk, const lora_weight *Wv,
                          WeightView &wq, WeightView &wk, WeightView &wv) {
  LORA_TRY(check_dims(dtype, T, k, nq, r));
  LORA_TRY(check_dims(dtype, T, k, nkv, r));
  LORA_TRY(check_weight(Wq, dtype, k, wq));
  LORA_TRY(check_weight(Wk, dtype, k, wk));
  LORA_TRY(check_weight(Wv, dtype, k, wv));
  if (dtype != LORA_BF16 || wq.q4 || wk.q4 || wv.q4) return LORA_ERR_UNSUPPORTED;
  if (!qkv_shapes_ok(k, nq, nkv, r)) return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

int lora_rmsnorm_qkv_fwd(int dtype, int64_t T, int64_t k, int64_t nq, int64_t nkv, int64_t r,
                         float alpha, float eps, const void *X, const void *norm_w,
                         const lora_weight *Wq, const void *Aq, const void *Bq,
                         const lora_weight *Wk, const void *Ak, const void *Bk,
                         const lora_weight *Wv, const void *Av, const void *Bv, void *Q, void *K,
                         void *V, float *rstd, void *ws, size_t ws_bytes, void *stream) {
  WeightView wq, wk, wv;
  LORA_TRY(check_qkv_norm(dtype, T, k, nq, nkv, r, Wq, Wk, Wv, wq, wk, wv));
  if (!(eps >= 0.f) || !std::isfinite(eps)) return LORA_ERR_UNSUPPORTED;
  LORA_TRY(check_ptrs({Aq, Bq, Ak, Bk, Av, Bv, norm_w}));
  LORA_TRY(check_tok_ptrs(T, {X, Q, K, V, rstd}));
  const size_t need = lora_qkv_workspace_bytes(LORA_OP_RMSNORM_QKV_FWD, dtype, LORA_W_DENSE, T, k,
                                               nq, nkv, r);
  if (ws_bytes < need) return LORA_ERR_WORKSPACE;
  if (need && (!ws || !aligned16(ws))) return ws ? LORA_ERR_MISALIGNED : LORA_ERR_NULL_POINTER;
  if (T == 0) return LORA_OK;
  const NormFuse nf{(const bf16_t *)norm_w, eps, rstd, false};
  return qkv_fwd_fused(T, k, nq, nkv, r, alpha, X, wq, wk, wv, Aq, Bq, Ak, Bk, Av, Bv, Q, K, V, ws,
                       (hipStream_t)stream, &nf);
}

int lora_rmsnorm_qkv_bwd(int dtype, int64_t T, int64_t k, int64_t nq, int64_t nkv, int64_t r,
                         float alpha, const void *X, const void *norm_w, const float *rstd,
                         const lora_weight *Wq, const void *Aq, const void *Bq,
                         const lora_weight *Wk, const void *Ak, const void *Bk,
                         const lora_weight *Wv, const void *Av, const void *Bv, const void *dQ,
                         const void *dK, const void *dV, void *dX, void *dAq, void *dBq,
                         void *dAk, void *dBk, void *dAv, void *dBv, uint32_t flags, void *ws,
                         size_t ws_bytes, void *stream) {
  WeightView wq, wk, wv;
  LORA_TRY(check_qkv_norm(dtype, T, k, nq, nkv, r, Wq, Wk, Wv, wq, wk, wv));
  LORA_TRY(check_ptrs({Aq, Bq, Ak, Bk, Av, Bv, dAq, dBq, dAk, dBk, dAv, dBv, norm_w}));
  LORA_TRY(check_tok_ptrs(T, {X, dQ, dK, dV, rstd}));
  if (dX && !aligned16(dX)) return LORA_ERR_MISALIGNED;
  if (flags & ~(uint32_t)LORA_FLAG_ACCUMULATE_DX) return LORA_ERR_UNSUPPORTED;
  const size_t need = lora_qkv_workspace_bytes(LORA_OP_RMSNORM_QKV_BWD, dtype, LORA_W_DENSE, T, k,
                                               nq, nkv, r);
  if (ws_bytes < need) return LORA_ERR_WORKSPACE;
  if (need && (!ws || !aligned16(ws))) return ws ? LORA_ERR_MISALIGNED : LORA_ERR_NULL_POINTER;
  const NormFuse nf{(const bf16_t *)norm_w, 0.f, const_cast<float *>(rstd),
                    (flags & LORA_FLAG_ACCUMULATE_DX) != 0};
  return qkv_bwd_fused(T, k, nq, nkv, r, alpha, X, wq, wk, wv, Aq, Bq, Ak, Bk, Av, Bv, dQ, dK, dV,
                       dX, dAq, dBq, dAk, dBk, dAv, dBv, nf.accumulate, ws, (hipStream_t)stream,
                       &nf);
}

int lora_merge(int dtype, int64_t n, int64_t k, int64_t r, float alpha, int sign,
               const lora_weight *W, const void *A, const void *B, void *out, void *stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_UNSUPPORTED;
  if (sign != 1 && sign != -1) return LORA_ERR_UNSUPPORTED;
  if (n <= 0 || k <= 0 || r <= 0 || n > ((int64_t)1 << 24) || k > ((int64_t)1 << 24))
    return LORA_ERR_BAD_SHAPE;
  if (r > LORA_MAX_RANK) return LORA_ERR_UNSUPPORTED;
  WeightView wv;
  LORA_TRY(check_weight(W, dtype, k, wv));
  LORA_TRY(check_ptrs({A, B, out}));
  const int64_t ncb = cdiv(k, 64), blocks = cdiv(n, 64) * ncb;
  if (blocks >= ((int64_t)1 << 31)) return LORA_ERR_BAD_SHAPE;
  MergeArgs a{(int)n, (int)k, (int)r, (int)ncb, (float)sign * (alpha / (float)r),
              dtype == LORA_F32, wv.q4 ? nullptr : (const void *)wv.w, wv.codes, wv.absmax,
              wv.codebook, A, B, out};
  hipLaunchKernelGGL(k_lora_merge, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
  HIP_TRY(hipGetLastError());
  return LORA_OK;
}

int lora_dequant4(int64_t n, int64_t k, const uint8_t *codes, const float *absmax,
                  const float *codebook, int blocksize, int out_dtype, void *out, void *stream) {
  if (!codes || !absmax || !codebook || !out) return LORA_ERR_NULL_POINTER;
  if (out_dtype != LORA_BF16 || blocksize != 64) return LORA_ERR_UNSUPPORTED;
  if (n <= 0 || k <= 0 || (k % 64) || n > ((int64_t)1 << 24) || k > ((int64_t)1 << 24) ||
      n * k > ((int64_t)1 << 44))
    return LORA_ERR_BAD_SHAPE;
  if (!aligned16(codes) || !aligned16(absmax) || !aligned16(codebook) || !aligned16(out))
    return LORA_ERR_MISALIGNED;
  const int64_t total = n * k;
  const AbsmaxSrc am{absmax, nullptr, nullptr, nullptr, 0.f};
  hipLaunchKernelGGL(k_dequant4, dim3(blocks_for(total / 32)), dim3(256), 0, (hipStream_t)stream,
                     codes, am, codebook, total, (bf16_t *)out);
  HIP_TRY(hipGetLastError());
  return LORA_OK;
}

int lora_rmsnorm_fwd(int dtype, int64_t T, int64_t d, float eps, const void *X, const void *w,
                     void *Y, float *rstd, void *stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_UNSUPPORTED;
  if (!(eps >= 0.f) || !std::isfinite(eps)) return LORA_ERR_UNSUPPORTED;
  if (T < 0 || d <= 0 || T > (int64_t)1 << 30 || d > (int64_t)1 << 24) return LORA_ERR_BAD_SHAPE;
  if (dtype == LORA_BF16 && (d % 8)) return LORA_ERR_BAD_SHAPE;
  LORA_TRY(check_ptrs({w}));
  LORA_TRY(check_tok_ptrs(T, {X, Y, rstd}));
  if (T == 0) return LORA_OK;
  const unsigned grid = (unsigned)cdiv(T, 4);
  if (dtype == LORA_F32)
    hipLaunchKernelGGL(k_rmsnorm_fwd<true>, dim3(grid), dim3(256), 0, (hipStream_t)stream, X, w,
                       eps, (int)T, (int)d, Y, rstd);
  else
    hipLaunchKernelGGL(k_rmsnorm_fwd<false>, dim3(grid), dim3(256), 0, (hipStream_t)stream, X, w,
                       eps, (int)T, (int)d, Y, rstd);
  HIP_TRY(hipGetLastError());
  return LORA_OK;
}

int lora_rmsnorm_bwd(int dtype, int64_t T, int64_t d, const void *X, const void *w,
                     const float *rstd, const void *dY, void *dX, uint32_t flags, void *stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_UNSUPPORTED;
  if (flags & ~LORA_FLAG_ACCUMULATE_DX) return LORA_ERR_UNSUPPORTED;
  if (T < 0 || d <= 0 || T > (int64_t)1 << 30 || d > (int64_t)1 << 24) return LORA_ERR_BAD_SHAPE;
  if (dtype == LORA_BF16 && (d % 8)) return LORA_ERR_BAD_SHAPE;
  LORA_TRY(check_ptrs({w}));
  LORA_TRY(check_tok_ptrs(T, {X, rstd, dY, dX}));
  if (T == 0) return LORA_OK;
  const unsigned grid = (unsigned)cdiv(T, 4);
  const int acc = (flags & LORA_FLAG_ACCUMULATE_DX) ? 1 : 0;
  if (dtype == LORA_F32)
    hipLaunchKernelGGL(k_rmsnorm_bwd<true>, dim3(grid), dim3(256), 0, (hipStream_t)stream, X, w,
                       rstd, dY, (int)T, (int)d, dX, acc);
  else
    hipLaunchKernelGGL(k_rmsnorm_bwd<false>, dim3(grid), dim3(256), 0, (hipStream_t)stream, X, w,
                       rstd, dY, (int)T, (int)d, dX, acc);
  HIP_TRY(hipGetLastError());
  return LORA_OK;
}

int lora_decode_weight(int64_t n, int64_t k, const lora_weight *W, int out_dtype, void *out,
                       void *stream) {
  if (out_dtype != LORA_BF16) return LORA_ERR_UNSUPPORTED;
  if (n <= 0 || k <= 0 || n > ((int64_t)1 << 24) || k > ((int64_t)1 << 24) ||
      n * k > ((int64_t)1 << 44))
    return LORA_ERR_BAD_SHAPE;
  if (!W) return LORA_ERR_NULL_POINTER;
  if (W->fmt == LORA_W_DENSE) return LORA_ERR_UNSUPPORTED;
  WeightView wv;
  LORA_TRY(check_weight(W, LORA_BF16, k, wv));
  LORA_TRY(check_ptrs({out}));
  return decode_w((bf16_t *)out, wv, n, k, (hipStream_t)stream);
}

}  // extern "C"
