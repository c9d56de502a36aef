// RMSNorm forward / backward over the rows of a [T x d] activation, the step
// in front of the gate/up and q/k/v projections ("Unsloth speed secrets:
// Triton kernels accelerate backprop", 3.2: per-row mean of squares, the
// reciprocal root kept for the backward, normalised row times the weight;
// "Unsloth code-reading guide", highlights: statistics in fp32, one cast
// back to the storage dtype at the end).
//
//   rstd[t] = 1 / sqrt(sum_j X[t,j]^2 / d + eps)              (fp32, saved)
//   Y[t,j]  = X[t,j] * rstd[t] * w[j]                         (fp32, rounded once)
//   dX[t,i] = rstd g_i - rstd^3 x_i (sum_j g_j x_j) / d,  g_j = dY[t,j] w[j]
//
// The weight w is frozen (no dw), as the base weights are.  One wave per
// row: a lane walks its 16-byte chunks in order and the wave adds the lane
// sums with a fixed butterfly, so results are bitwise reproducible.  Both
// kernels are HBM-bound; rows up to d = 8192 (forward) / 4096 (backward) are
// read once and kept in registers for the second pass.
#pragma once
#include "common.hpp"

namespace lora {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ void unpack8(const u32x4 &v, float o[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = bf16lo(v[i]);
    o[2 * i + 1] = bf16hi(v[i]);
  }
}

// bf16 rows (d % 8 == 0) move as 16-byte chunks; rows of up to kRegChunks x 64
// chunks (d <= 8192) stay in registers between the two passes, longer rows
// are read again (from L2).  fp32 rows go element by element.
constexpr int kRegChunks = 16;

template <bool F32>
__global__ __launch_bounds__(256) void k_rmsnorm_fwd(const void *Xv, const void *wv, float eps,
                                                     int T, int d, void *Yv, float *rstd) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  if constexpr (F32) {
    const float *x = reinterpret_cast<const float *>(Xv) + (int64_t)row * d;
    const float *w = reinterpret_cast<const float *>(wv);
    float *y = reinterpret_cast<float *>(Yv) + (int64_t)row * d;
    float ss = 0.f;
    for (int j = lane; j < d; j += 64) ss = fmaf(x[j], x[j], ss);
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    if (lane == 0) rstd[row] = r;
    for (int j = lane; j < d; j += 64) y[j] = x[j] * r * w[j];
  } else {
    const bf16_t *x = reinterpret_cast<const bf16_t *>(Xv) + (int64_t)row * d;
    const bf16_t *w = reinterpret_cast<const bf16_t *>(wv);
    bf16_t *y = reinterpret_cast<bf16_t *>(Yv) + (int64_t)row * d;
    const int nch = d / 8;
    const bool resident = nch <= 64 * kRegChunks;
    u32x4 xr[kRegChunks];
    float ss = 0.f;
    auto add_sq = [&](const u32x4 &c) {
      float v[8];
      unpack8(c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
    };
    if (resident) {
#pragma unroll
      for (int i = 0; i < kRegChunks; ++i)
        if (lane + 64 * i < nch) xr[i] = gload16(x + 8 * (lane + 64 * i));
#pragma unroll
      for (int i = 0; i < kRegChunks; ++i)
        if (lane + 64 * i < nch) add_sq(xr[i]);
    } else {
      for (int c = lane; c < nch; c += 64) add_sq(gload16(x + 8 * c));
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    if (lane == 0) rstd[row] = r;
    if (Yv == nullptr) return;   // statistics only (the norm folded into the projections)
    auto out = [&](int c, const u32x4 &xc) {
      float v[8], g[8];
      unpack8(xc, v);
      unpack8(gload16(w + 8 * c), g);
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = pack_bf16x2(v[2 * i] * r * g[2 * i], v[2 * i + 1] * r * g[2 * i + 1]);
      gstore16(y + 8 * c, o);
    };
    if (resident) {
#pragma unroll
      for (int i = 0; i < kRegChunks; ++i)
        if (lane + 64 * i < nch) out(lane + 64 * i, xr[i]);
    } else {
      for (int c = lane; c < nch; c += 64) out(c, gload16(x + 8 * c));
    }
  }
}

// dX = (or +=, accumulate != 0) the input gradient of k_rmsnorm_fwd; wv
// NULL stands for a unit weight (dY is then already the gradient with
// respect to X rstd diag(w), as a folded projection returns it)
template <bool F32>
__global__ __launch_bounds__(256) void k_rmsnorm_bwd(const void *Xv, const void *wv,
                                                     const float *rstd, const void *dYv, int T,
                                                     int d, void *dXv, int accumulate) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const float r = rstd[row];
  if constexpr (F32) {
    const float *x = reinterpret_cast<const float *>(Xv) + (int64_t)row * d;
    const float *w = reinterpret_cast<const float *>(wv);
    const float *dy = reinterpret_cast<const float *>(dYv) + (int64_t)row * d;
    float *dx = reinterpret_cast<float *>(dXv) + (int64_t)row * d;
    float dot = 0.f;
    for (int j = lane; j < d; j += 64) dot = fmaf(dy[j] * (w ? w[j] : 1.f), x[j], dot);
    dot = wave_sum(dot);
    const float cx = r * r * r * dot / (float)d;   // coefficient of x_i
    for (int j = lane; j < d; j += 64) {
      const float v = r * (dy[j] * (w ? w[j] : 1.f)) - cx * x[j];
      dx[j] = accumulate ? dx[j] + v : v;
    }
  } else {
    const bf16_t *x = reinterpret_cast<const bf16_t *>(Xv) + (int64_t)row * d;
    const bf16_t *w = reinterpret_cast<const bf16_t *>(wv);
    const bf16_t *dy = reinterpret_cast<const bf16_t *>(dYv) + (int64_t)row * d;
    bf16_t *dx = reinterpret_cast<bf16_t *>(dXv) + (int64_t)row * d;
    const int nch = d / 8;
    // x and dy of rows up to half the register budget stay resident
    constexpr int RC = kRegChunks / 2;
    const bool resident = nch <= 64 * RC;
    u32x4 xr[RC], gr[RC];
    float dot = 0.f;
    auto wload = [&](int c, float *wv8) {
      if (w) {
        unpack8(gload16(w + 8 * c), wv8);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) wv8[i] = 1.f;
      }
    };
    auto add_dot = [&](int c, const u32x4 &xc, const u32x4 &gc) {
      float xv[8], wv8[8], gv[8];
      unpack8(xc, xv);
      wload(c, wv8);
      unpack8(gc, gv);
#pragma unroll
      for (int i = 0; i < 8; ++i) dot = fmaf(gv[i] * wv8[i], xv[i], dot);
    };
    if (resident) {
#pragma unroll
      for (int i = 0; i < RC; ++i)
        if (lane + 64 * i < nch) {
          xr[i] = gload16(x + 8 * (lane + 64 * i));
          gr[i] = gload16(dy + 8 * (lane + 64 * i));
        }
#pragma unroll
      for (int i = 0; i < RC; ++i)
        if (lane + 64 * i < nch) add_dot(lane + 64 * i, xr[i], gr[i]);
    } else {
      for (int c = lane; c < nch; c += 64) add_dot(c, gload16(x + 8 * c), gload16(dy + 8 * c));
    }
    dot = wave_sum(dot);
    const float cx = r * r * r * dot / (float)d;   // coefficient of x_i
    auto out = [&](int c, const u32x4 &xc, const u32x4 &gc) {
      float xv[8], wv8[8], gv[8], o8[8];
      unpack8(xc, xv);
      wload(c, wv8);
      unpack8(gc, gv);
#pragma unroll
      for (int i = 0; i < 8; ++i) o8[i] = r * (gv[i] * wv8[i]) - cx * xv[i];
      if (accumulate) {
        float old[8];
        unpack8(gload16(dx + 8 * c), old);
#pragma unroll
        for (int i = 0; i < 8; ++i) o8[i] += old[i];
      }
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(o8[2 * i], o8[2 * i + 1]);
      gstore16(dx + 8 * c, o);
    };
    if (resident) {
#pragma unroll
      for (int i = 0; i < RC; ++i)
        if (lane + 64 * i < nch) out(lane + 64 * i, xr[i], gr[i]);
    } else {
      for (int c = lane; c < nch; c += 64) out(c, gload16(x + 8 * c), gload16(dy + 8 * c));
    }
  }
}

}  // namespace lora
