// bf16 MFMA GEMM with a fused LoRA branch, for gfx950.
//
//   C[M x N] = A_op[M x K] . B_op^T  +  s * S[M x RS] . E[N x RS]^T
//
// where the rank-r side product S = A_op . SIDE^T is accumulated inside the
// same K loop from the A tile already staged in LDS (it is never written to
// memory, "Why Unsloth trains 5-8x faster", section 3.2: x_a stays on chip),
// rounded to bf16 after scaling by s, and applied in the epilogue as a second
// MFMA pass with K = RS.  RS is the rank padded to a multiple of 16.
//
// Operand B comes in four forms:
//   B_NT     dense [N x K] rows (forward: W of an nn.Linear, K-contiguous)
//   B_NT_Q4  4-bit codes of the same [N x K] weight, decoded while filling LDS
//   B_NN     dense [K x N] rows (backward dX = dY W: W is N-contiguous); the
//            loader transposes 8x8 bf16 blocks in registers before the LDS
//            write, so both layouts share one LDS format and one MFMA loop
//   B_NN_Q4  4-bit codes of the [K x N] weight, decoded then transposed
// The 4-bit decode is bf16_rne(codebook[c] * absmax) with one fp32 multiply
// ("Unsloth code-reading guide", section 2.1: 4-bit weights are decoded to
// bf16 before every matmul; "Why Unsloth trains 5-8x faster", section 5.2:
// decode fused into the matmul).
//
// Epilogues:
//   EPI_STORE       C (bf16), optionally accumulating into C
//   EPI_SWIGLU_FWD  gate/up interleaved tile: e, g, h = silu(e) g (bf16)
//   EPI_SWIGLU_BWD  dh tile: loads saved e, g; writes de, dg (bf16)
//
// Tile: 256 x 256 x 64, 256 threads = 4 waves in a 2 x 2 grid, each wave a
// 128 x 128 sub-tile of 4 x 4 MFMA 32x32x16 blocks.  The MFMA "A" operand is
// the B_op fragment and the "B" operand the A_op fragment, so each lane ends
// with 4 consecutive output columns of one output row (8-byte stores).
// LDS: two stages of {A tile 32 KB, B tile 32 KB, SIDE tile RS x 64}.
#pragma once
#include "common.hpp"

namespace lora {

constexpr int BM = 256, BN = 256, BK = 64, NTHREADS = 256;

enum BMode { B_NT = 0, B_NT_Q4 = 1, B_NN = 2, B_NN_Q4 = 3 };
enum Epi { EPI_STORE = 0, EPI_SWIGLU_FWD = 1, EPI_SWIGLU_BWD = 2 };
// side modes: where the rank-r product comes from
enum SideMode { SIDE_INLOOP = 1, SIDE_GLOBAL = 2 };

struct GemmArgs {
  int M, N, K;
  int ksplit;                   // K index where A0/B0 hand over to A1/B1
  const bf16_t *A0, *A1;        // A_op rows, K-contiguous
  int64_t lda;
  const bf16_t *B0, *B1;        // dense B_op
  int64_t ldb;                  // NT: row stride (>= K); NN: row stride (>= N)
  const uint8_t *Q0, *Q1;       // 4-bit codes
  const float *S0, *S1;         // 4-bit absmax
  const float *codebook;        // 16 fp32 levels
  int gu_f;                     // SwiGLU forward: feature count f (N = 2 f)
  const bf16_t *side;           // SIDE_INLOOP: [RS x K] bf16, zero padded
  int64_t ld_side;
  const bf16_t *hglob;          // SIDE_GLOBAL: s * S precomputed, [M x rs] bf16
  int rs;                       // side width (multiple of 16)
  const bf16_t *epi;            // [rows x rs] bf16 epilogue LoRA operand
  float s;
  int accumulate;               // EPI_STORE: C += result
  bf16_t *C;
  int64_t ldc;
  bf16_t *E, *G, *H;            // SwiGLU forward outputs [M x f]
  const bf16_t *Ein, *Gin;      // SwiGLU backward saved activations [M x N]
  bf16_t *DE, *DG;              // SwiGLU backward outputs [M x N]
  float *side_out;              // [M x rs] fp32 unscaled side product (nullable)
  int tiles_m, tiles_n;
};

// XCD-aware, grouped tile order.  Workgroups are dispatched round-robin over
// the 8 XCDs; remapping gives each XCD a contiguous run of logical tiles, and
// the grouped order makes the ~32 tiles resident on one XCD share 4 row
// blocks of A_op and 8 column blocks of B_op in that XCD's L2.
__device__ __forceinline__ void map_tile(int bid, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int nwg = tiles_m * tiles_n;
  int logical = bid;
  if ((nwg & 7) == 0) logical = (bid & 7) * (nwg >> 3) + (bid >> 3);
  constexpr int GM = 4;
  const int group = logical / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int in_group = logical - group * GM * tiles_n;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

template <int BMODE, int RS, int SMODE>
struct Stage {
  u32x4 xa[8];
  u32x4 wb[(BMODE == B_NT || BMODE == B_NN) ? 8 : 1];
  u32x4 qc[(BMODE == B_NT_Q4) ? 2 : 1];
  uint32_t qn[(BMODE == B_NN_Q4) ? 8 : 1];
  float qs[(BMODE == B_NN_Q4) ? 8 : 1];
  u32x4 sd[(SMODE == SIDE_INLOOP && RS * 8 > NTHREADS) ? (RS * 8 / NTHREADS) : 1];
};

template <int BMODE, int RS, int EPI, int SMODE>
__global__ __launch_bounds__(NTHREADS, 1) void k_lora_gemm(const GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr bool GU = (EPI == EPI_SWIGLU_FWD);
  constexpr bool Q4 = (BMODE == B_NT_Q4 || BMODE == B_NN_Q4);
  constexpr bool NN = (BMODE == B_NN || BMODE == B_NN_Q4);
  constexpr bool INLOOP = (SMODE == SIDE_INLOOP);
  constexpr int XS = BM * BK * 2, WS = BN * BK * 2;
  constexpr int SS = INLOOP ? RS * BK * 2 : 0;
  constexpr int STAGE = XS + WS + SS;
  constexpr int NSB = INLOOP ? RS / 16 : 1;   // side row blocks of 16

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi32 = lane >> 5;
  const int l16 = lane & 15, hi16 = lane >> 4;

  int tm, tn;
  map_tile(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K;

  float2 *cbt = reinterpret_cast<float2 *>(smem + 2 * STAGE);   // 4-bit pair table
  if constexpr (Q4) {
    // entry b = (codebook[b & 15], codebook[b >> 4]): a code byte decodes
    // into its two elements with one LDS read
    cbt[tid] = make_float2(p.codebook[tid & 15], p.codebook[tid >> 4]);
  }

  // ------------------------------------------------ global -> registers
  auto load_stage = [&](Stage<BMODE, RS, SMODE> &st, int kt) {
    const int k0 = kt * BK;
    // A_op tile: 256 rows x 8 chunks, thread takes chunk (tid&7) of 8 rows
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (tid >> 3) + 32 * i, c = tid & 7;
      const int gm = m0 + row, gk = k0 + c * 8;
      u32x4 v = {0, 0, 0, 0};
      if (gm < M && gk < K) {
        const bf16_t *src = gk < p.ksplit ? p.A0 + (int64_t)gm * p.lda + gk
                                          : p.A1 + (int64_t)gm * p.lda + (gk - p.ksplit);
        v = gload16(src);
      }
      st.xa[i] = v;
    }
    if constexpr (BMODE == B_NT) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = (tid >> 3) + 32 * i, c = tid & 7;
        const int gk = k0 + c * 8;
        u32x4 v = {0, 0, 0, 0};
        if constexpr (GU) {
          const int half = row >> 7, sub = row & 127;
          const int j = tn * 128 + half * 64 + (sub & 63);
          if (j < p.gu_f && gk < K)
            v = gload16(((sub >> 6) ? p.B1 : p.B0) + (int64_t)j * p.ldb + gk);
        } else {
          const int gn = n0 + row;
          if (gn < N && gk < K) v = gload16(p.B0 + (int64_t)gn * p.ldb + gk);
        }
        st.wb[i] = v;
      }
    } else if constexpr (BMODE == B_NT_Q4) {
      // one weight row per thread: 64 codes (32 bytes) + one absmax (K % 64 == 0)
      const int row = tid;
      int64_t grow = -1;
      const uint8_t *q = p.Q0;
      const float *sc = p.S0;
      if constexpr (GU) {
        const int half = row >> 7, sub = row & 127;
        const int j = tn * 128 + half * 64 + (sub & 63);
        if (j < p.gu_f) grow = j;
        if (sub >> 6) { q = p.Q1; sc = p.S1; }
      } else {
        if (n0 + row < N) grow = n0 + row;
      }
      u32x4 c0 = {0, 0, 0, 0}, c1 = {0, 0, 0, 0};
      float am = 0.f;
      if (grow >= 0) {
        const uint8_t *src = q + grow * (int64_t)(K / 2) + k0 / 2;
        c0 = gload16(src);
        c1 = gload16(src + 16);
        am = sc[(grow * (int64_t)K + k0) >> 6];
      }
      st.qc[0] = c0;
      st.qc[1] = c1;
      st.qs[0] = am;
    } else if constexpr (BMODE == B_NN) {
      const int kb = tid >> 5, nb = tid & 31;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int gk = k0 + kb * 8 + i, gn = n0 + nb * 8;
        u32x4 v = {0, 0, 0, 0};
        if (gk < K && gn < N) {
          const bf16_t *src = gk < p.ksplit ? p.B0 + (int64_t)gk * p.ldb + gn
                                            : p.B1 + (int64_t)(gk - p.ksplit) * p.ldb + gn;
          v = gload16(src);
        }
        st.wb[i] = v;
      }
    } else {  // B_NN_Q4: weight rows gk, 8 columns gn.. (4 bytes of codes)
      const int kb = tid >> 5, nb = tid & 31;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int gk = k0 + kb * 8 + i, gn = n0 + nb * 8;
        uint32_t cw = 0;
        float am = 0.f;
        if (gk < K && gn < N) {
          const bool first = gk < p.ksplit;
          const int64_t wr = first ? gk : gk - p.ksplit;
          const uint8_t *q = first ? p.Q0 : p.Q1;
          const float *sc = first ? p.S0 : p.S1;
          cw = *reinterpret_cast<const uint32_t *>(q + wr * (int64_t)(N / 2) + gn / 2);
          am = sc[(wr * (int64_t)N + gn) >> 6];
        }
        st.qn[i] = cw;
        st.qs[i] = am;
      }
    }
    if constexpr (INLOOP) {
#pragma unroll
      for (int u = 0; u < (RS * 8 + NTHREADS - 1) / NTHREADS; ++u) {
        const int q = tid + NTHREADS * u;
        const int row = q >> 3, c = q & 7;
        const int gk = k0 + c * 8;
        u32x4 v = {0, 0, 0, 0};
        if (row < RS && gk < K) v = gload16(p.side + (int64_t)row * p.ld_side + gk);
        st.sd[u] = v;
      }
    }
  };

  // 4 code bytes (8 elements) -> 8 bf16 packed in 4 words
  auto decode4 = [&](uint32_t cw, float am) -> u32x4 {
    u32x4 o;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float2 cv = cbt[(cw >> (8 * b)) & 0xFFu];
      o[b] = pack_bf16x2(cv.x * am, cv.y * am);
    }
    return o;
  };

  // ------------------------------------------------ registers -> LDS
  auto store_stage = [&](Stage<BMODE, RS, SMODE> &st, char *stage) {
    char *Xs = stage, *Ws = stage + XS, *Ss = stage + XS + WS;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      lds_write16(Xs, swz_off((tid >> 3) + 32 * i, tid & 7), st.xa[i]);
    if constexpr (BMODE == B_NT) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        lds_write16(Ws, swz_off((tid >> 3) + 32 * i, tid & 7), st.wb[i]);
    } else if constexpr (BMODE == B_NT_Q4) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const u32x4 &src = st.qc[c >> 2];
        lds_write16(Ws, swz_off(tid, c), decode4(src[c & 3], st.qs[0]));
      }
    } else {
      u32x4 rows[8], cols[8];
      const int kb = tid >> 5, nb = tid & 31;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (BMODE == B_NN) rows[i] = st.wb[i];
        else rows[i] = decode4(st.qn[i], st.qs[i]);
      }
      transpose8x8(rows, cols);
#pragma unroll
      for (int j = 0; j < 8; ++j) lds_write16(Ws, swz_off(nb * 8 + j, kb), cols[j]);
    }
    if constexpr (INLOOP) {
#pragma unroll
      for (int u = 0; u < (RS * 8 + NTHREADS - 1) / NTHREADS; ++u) {
        const int q = tid + NTHREADS * u;
        if (q < RS * 8) lds_write16(Ss, swz_off(q >> 3, q & 7), st.sd[u]);
      }
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  f32x4 sacc[NSB][4];
#pragma unroll
  for (int a = 0; a < NSB; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) sacc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nkt = (K + BK - 1) / BK;
  Stage<BMODE, RS, SMODE> st;
  if (Q4) __syncthreads();  // pair table visible before the first decode
  load_stage(st, 0);
  store_stage(st, smem);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const char *cur = smem + (kt & 1) * STAGE;
    if (kt + 1 < nkt) load_stage(st, kt + 1);
    {
      const char *Xs = cur, *Ws = cur + XS;
      u32x4 fa[2][4], fb[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[0][i] = lds_read16(Ws, swz_off(wn * 128 + i * 32 + l32, hi32));
        fb[0][i] = lds_read16(Xs, swz_off(wm * 128 + i * 32 + l32, hi32));
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int cb = kk & 1, nb = cb ^ 1;
        if (kk < 3) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            fa[nb][i] = lds_read16(Ws, swz_off(wn * 128 + i * 32 + l32, 2 * (kk + 1) + hi32));
            fb[nb][i] = lds_read16(Xs, swz_off(wm * 128 + i * 32 + l32, 2 * (kk + 1) + hi32));
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fa[cb][i], fb[cb][j], acc[i][j]);
      }
      if constexpr (INLOOP) {
        const char *Ss = cur + XS + WS;
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
          u32x4 sa[NSB], xb[4];
#pragma unroll
          for (int sb = 0; sb < NSB; ++sb)
            sa[sb] = lds_read16(Ss, swz_off(sb * 16 + l16, 4 * kq + hi16));
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
            xb[mb] = lds_read16(Xs, swz_off(wm * 128 + wn * 64 + mb * 16 + l16, 4 * kq + hi16));
#pragma unroll
          for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) sacc[sb][mb] = mfma16(sa[sb], xb[mb], sacc[sb][mb]);
        }
      }
    }
    if (kt + 1 < nkt) store_stage(st, smem + ((kt + 1) & 1) * STAGE);
    __syncthreads();
  }

  // ------------------------------------------------ LoRA epilogue pass
  const int rs = INLOOP ? RS : p.rs;
  const int rs_bytes = rs * 2;
  const char *Hl = smem;
  if constexpr (INLOOP) {
    // bf16(s * S) into LDS rows [m_local][rs]; fp32 S to side_out if asked
    char *Hw = smem;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int ml = wm * 128 + wn * 64 + mb * 16 + l16;
        const int q = sb * 16 + 4 * hi16;
        const f32x4 v = sacc[sb][mb];
        u32x2 w = {pack_bf16x2(p.s * v[0], p.s * v[1]), pack_bf16x2(p.s * v[2], p.s * v[3])};
        *reinterpret_cast<u32x2 *>(Hw + ml * rs_bytes + q * 2) = w;
        if (p.side_out != nullptr && tn == 0 && m0 + ml < M)
          *reinterpret_cast<f32x4 *>(p.side_out + (int64_t)(m0 + ml) * RS + q) = v;
      }
    __syncthreads();
  }
  for (int kq = 0; kq < rs / 16; ++kq) {
    u32x4 ea[4], hb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t erow;
      bool ok;
      if constexpr (GU) {
        const int j = tn * 128 + wn * 64 + (i & 1) * 32 + l32;
        ok = j < p.gu_f;
        erow = (i >= 2 ? p.gu_f : 0) + j;
      } else {
        const int n = n0 + wn * 128 + i * 32 + l32;
        ok = n < N;
        erow = n;
      }
      u32x4 v = {0, 0, 0, 0};
      if (ok) v = gload16(p.epi + erow * rs + kq * 16 + 8 * hi32);
      ea[i] = v;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ml = wm * 128 + j * 32 + l32;
      if constexpr (INLOOP) {
        hb[j] = lds_read16(Hl, ml * rs_bytes + (kq * 16 + 8 * hi32) * 2);
      } else {
        u32x4 v = {0, 0, 0, 0};
        if (m0 + ml < M) v = gload16(p.hglob + (int64_t)(m0 + ml) * rs + kq * 16 + 8 * hi32);
        hb[j] = v;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(ea[i], hb[j], acc[i][j]);
  }

  // ------------------------------------------------ output
  if constexpr (EPI == EPI_STORE) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm * 128 + j * 32 + l32;
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * 128 + i * 32 + 8 * g + 4 * hi32;
          if (n >= N) continue;
          float v0 = acc[i][j][4 * g], v1 = acc[i][j][4 * g + 1];
          float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
          bf16_t *dst = p.C + (int64_t)m * p.ldc + n;
          if (p.accumulate) {
            const u32x2 o = gload8(dst);
            v0 += bf16lo(o[0]); v1 += bf16hi(o[0]);
            v2 += bf16lo(o[1]); v3 += bf16hi(o[1]);
          }
          gstore8(dst, u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)});
        }
    }
  } else if constexpr (EPI == EPI_SWIGLU_FWD) {
    const int f = p.gu_f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm * 128 + j * 32 + l32;
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int jf = tn * 128 + wn * 64 + i * 32 + 8 * g + 4 * hi32;
          if (jf >= f) continue;
          uint32_t ew[2], gw[2], hw[2];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            ew[h2] = pack_bf16x2(acc[i][j][4 * g + 2 * h2], acc[i][j][4 * g + 2 * h2 + 1]);
            gw[h2] = pack_bf16x2(acc[i + 2][j][4 * g + 2 * h2], acc[i + 2][j][4 * g + 2 * h2 + 1]);
            // h from the rounded e, g: the same values the backward reloads
            const float e0 = bf16lo(ew[h2]), e1 = bf16hi(ew[h2]);
            const float g0 = bf16lo(gw[h2]), g1 = bf16hi(gw[h2]);
            hw[h2] = pack_bf16x2(e0 * sigmoidf_fast(e0) * g0, e1 * sigmoidf_fast(e1) * g1);
          }
          const int64_t off = (int64_t)m * f + jf;
          gstore8(p.E + off, u32x2{ew[0], ew[1]});
          gstore8(p.G + off, u32x2{gw[0], gw[1]});
          gstore8(p.H + off, u32x2{hw[0], hw[1]});
        }
    }
  } else {  // EPI_SWIGLU_BWD
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm * 128 + j * 32 + l32;
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * 128 + i * 32 + 8 * g + 4 * hi32;
          if (n >= N) continue;
          const int64_t off = (int64_t)m * N + n;
          const u32x2 ev = gload8(p.Ein + off), gv = gload8(p.Gin + off);
          uint32_t dew[2], dgw[2];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            float de[2], dg[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const float e = t ? bf16hi(ev[h2]) : bf16lo(ev[h2]);
              const float gg = t ? bf16hi(gv[h2]) : bf16lo(gv[h2]);
              const float dh = acc[i][j][4 * g + 2 * h2 + t];
              const float sg = sigmoidf_fast(e);
              dg[t] = dh * e * sg;
              de[t] = dh * gg * sg * (1.0f + e * (1.0f - sg));
            }
            dew[h2] = pack_bf16x2(de[0], de[1]);
            dgw[h2] = pack_bf16x2(dg[0], dg[1]);
          }
          gstore8(p.DE + off, u32x2{dew[0], dew[1]});
          gstore8(p.DG + off, u32x2{dgw[0], dgw[1]});
        }
    }
  }
}

template <int BMODE, int RS, int EPI, int SMODE>
constexpr size_t gemm_lds_bytes() {
  return 2 * (size_t)(BM * BK * 2 + BN * BK * 2 + (SMODE == SIDE_INLOOP ? RS * BK * 2 : 0)) +
         ((BMODE == B_NT_Q4 || BMODE == B_NN_Q4) ? 256 * sizeof(float2) : 0);
}

}  // namespace lora
