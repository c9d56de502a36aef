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

// Instruction-scheduling groups (masks: 0x008 MFMA, 0x100 LDS read).
template <int MASK, int COUNT>
__device__ __forceinline__ void sched_group() {
  if constexpr (COUNT > 0) __builtin_amdgcn_sched_group_barrier(MASK, COUNT, 0);
}
// COUNT pairs of (one MFMA, one LDS read)
template <int COUNT>
__device__ __forceinline__ void sched_pairs() {
#pragma unroll
  for (int i = 0; i < COUNT; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// NN weight tiles are kept in their natural [64 K-rows x 256 N-cols] layout
// (512-byte rows); the 16-byte chunk index is XORed with 4 (row % 4) so the
// four rows one 16-lane group reads with ds_read_b64_tr_b16 fall in
// different banks.
__device__ __forceinline__ uint32_t nn_off(uint32_t row, uint32_t chunk) {
  return row * 512u + ((chunk ^ ((row & 3u) << 2)) << 4);
}

template <int BMODE>
struct Stage {
  // register-staged B operand (the DMA-loaded forms keep nothing here)
  u32x4 qc[(BMODE == B_NT_Q4) ? 2 : 1];
  uint32_t qn[(BMODE == B_NN_Q4) ? 8 : 1];
  float qs[(BMODE == B_NN_Q4) ? 8 : 1];
};

template <int BMODE, int RS, int EPI, int SMODE>
__global__ __launch_bounds__(NTHREADS, 1) void k_lora_gemm(const GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr bool GU = (EPI == EPI_SWIGLU_FWD);
  constexpr bool Q4 = (BMODE == B_NT_Q4 || BMODE == B_NN_Q4);
  constexpr bool INLOOP = (SMODE == SIDE_INLOOP);
  constexpr bool NN = (BMODE == B_NN || BMODE == B_NN_Q4);
  constexpr int XS = BM * BK * 2, WS = BN * BK * 2;
  constexpr int SS = INLOOP ? RS * BK * 2 : 0;
  constexpr int STAGE = XS + WS + SS;
  constexpr int NSB = INLOOP ? RS / 16 : 1;   // side row blocks of 16

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi32 = lane >> 5;
  const int l16 = lane & 15, hi16 = lane >> 4;

  int tm, tn;
  map_tile(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K, ksplit = p.ksplit;

  float2 *cbt = reinterpret_cast<float2 *>(smem + 2 * STAGE);   // 4-bit pair table
  if constexpr (Q4) {
    // entry b = (codebook[b & 15], codebook[b >> 4]): a code byte decodes
    // into its two elements with one LDS read
    cbt[tid] = make_float2(p.codebook[tid & 15], p.codebook[tid >> 4]);
  }

  // ---------------------------------------------------- DMA lane geometry
  // DMA instruction u of wave w fills tile rows 8b..8b+7 (b = 4u + w); lane
  // l lands in row 8b + l/8 at LDS chunk l%8, which holds logical K chunk
  // c = (l%8) ^ swz(row) = (l%8) ^ (l/8) ^ (b%8).
  const int lr = lane >> 3;
  const int c0 = (lane & 7) ^ lr;
  // A_op: byte offsets relative to row m0 (kOOB for rows past M)
  const bf16_t *Abase = p.A0 + (int64_t)m0 * p.lda;
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(Abase, kMaxRecords);
  // A1 - A0 - 2 ksplit: added to offsets of columns >= ksplit
  const uint32_t dA1 = (uint32_t)((const char *)p.A1 - (const char *)p.A0) - 2u * (uint32_t)ksplit;
  uint32_t aoff[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int b = 4 * u + wave, row = 8 * b + lr, c = c0 ^ (b & 7);
    aoff[u] = (m0 + row < M) ? (uint32_t)(row * p.lda * 2 + c * 16) : kOOB;
  }
  uint32_t boff[8];
  __amdgpu_buffer_rsrc_t rsB0, rsB1;
  if constexpr (BMODE == B_NT) {
    if constexpr (GU) {
      rsB0 = make_rsrc(p.B0 + (int64_t)tn * 128 * p.ldb, kMaxRecords);
      rsB1 = make_rsrc(p.B1 + (int64_t)tn * 128 * p.ldb, kMaxRecords);
    } else {
      rsB0 = rsB1 = make_rsrc(p.B0 + (int64_t)n0 * p.ldb, kMaxRecords);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int b = 4 * u + wave, row = 8 * b + lr, c = c0 ^ (b & 7);
      if constexpr (GU) {
        const int jl = (row >> 7) * 64 + (row & 63);
        boff[u] = (tn * 128 + jl < p.gu_f) ? (uint32_t)(jl * p.ldb * 2 + c * 16) : kOOB;
      } else {
        boff[u] = (n0 + row < N) ? (uint32_t)(row * p.ldb * 2 + c * 16) : kOOB;
      }
    }
  } else if constexpr (BMODE == B_NN) {
    // DMA instruction u of wave w fills K-rows 2b, 2b+1 (b = 4u + w); lane l
    // lands in row 2b + l/32 at 16-byte chunk l%32, holding logical chunk
    // (l%32) ^ 4 (row%4).  Rows >= ksplit come from B1.
    rsB0 = make_rsrc(p.B0 + n0, kMaxRecords);
    rsB1 = make_rsrc(p.B1 + n0, kMaxRecords);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int b = 4 * u + wave, row = 2 * b + (lane >> 5);
      const int c = (lane & 31) ^ ((row & 3) << 2);
      boff[u] = (n0 + 8 * c < N) ? (uint32_t)((lane >> 5) * p.ldb * 2 + c * 16) : kOOB;
    }
  } else if constexpr (BMODE == B_NT_Q4) {
    // one weight row per thread; gate rows for waves 0, 2 and up rows for
    // waves 1, 3 when the tile interleaves gate/up
    const int row = tid;
    int jl = row, jg = n0 + row;
    bool up = false;
    if constexpr (GU) {
      jl = (row >> 7) * 64 + (row & 63);
      jg = tn * 128 + jl;
      up = (row >> 6) & 1;
    }
    const int64_t grow0 = GU ? (int64_t)tn * 128 : (int64_t)n0;
    const uint8_t *q = up ? p.Q1 : p.Q0;
    const float *sc = up ? p.S1 : p.S0;
    rsB0 = make_rsrc(q + grow0 * (K / 2), kMaxRecords);
    rsB1 = make_rsrc(sc + grow0 * (K / 64), kMaxRecords);
    const bool ok = GU ? (jg < p.gu_f) : (jg < N);
    boff[0] = ok ? (uint32_t)(jl * (K / 2)) : kOOB;       // codes
    boff[1] = ok ? (uint32_t)(jl * (K / 64) * 4) : kOOB;  // absmax
  }
  // NN: byte offset of this lane's transpose-read row for n-block i at
  // K sub-step 0 (rows kk*16 + 4t are reached with immediate offsets)
  uint32_t trb[4];
  if constexpr (NN) {
    const int g = lane >> 4, sl = lane & 15;
    const int krow0 = 8 * (g >> 1) + (sl >> 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int nl = wn * 128 + i * 32 + 16 * (g & 1) + 4 * (sl & 3);
      trb[i] = nn_off(krow0, nl >> 3) + ((nl >> 2) & 1) * 8;
    }
  }
  uint32_t soff_side[(RS / 8 + 3) / 4];
  __amdgpu_buffer_rsrc_t rsS;
  if constexpr (INLOOP) {
    rsS = make_rsrc(p.side, kMaxRecords);
#pragma unroll
    for (int u = 0; u < (RS / 8 + 3) / 4; ++u) {
      const int b = 4 * u + wave, row = 8 * b + lr, c = c0 ^ (b & 7);
      soff_side[u] = (uint32_t)(row * p.ld_side * 2 + c * 16);
    }
  }

  // ------------------------------------------------ K tile kt -> stage
  // Issues the DMA loads of tile kt into `stage` and fills the register
  // staging of the non-DMA operand forms.
  auto issue_tile = [&](Stage<BMODE> &st, int kt, char *stage) {
    const int k0 = kt * BK;
    char *Xs = stage, *Ws = stage + XS, *Ss = stage + XS + WS;
    const bool full = (k0 + BK <= K) && (k0 + BK <= ksplit || k0 >= ksplit);
    if (full) {
      const uint32_t sa = 2u * (uint32_t)k0 + (k0 >= ksplit ? dA1 : 0u);
#pragma unroll
      for (int u = 0; u < 8; ++u) dma16(rsA, Xs + (4 * u + wave) * 1024, aoff[u], sa);
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int b = 4 * u + wave, col = k0 + 8 * (c0 ^ (b & 7));
        const uint32_t v = (aoff[u] != kOOB && col < K)
                               ? aoff[u] + 2u * (uint32_t)k0 + (col >= ksplit ? dA1 : 0u)
                               : kOOB;
        dma16(rsA, Xs + b * 1024, v, 0);
      }
    }
    const bool kfull = k0 + BK <= K;
    if constexpr (BMODE == B_NT) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int b = 4 * u + wave;
        const __amdgpu_buffer_rsrc_t r = (GU && ((b >> 3) & 1)) ? rsB1 : rsB0;
        uint32_t v = boff[u];
        if (!kfull) {
          const int col = k0 + 8 * (c0 ^ (b & 7));
          if (col >= K) v = kOOB;
        }
        dma16(r, Ws + b * 1024, v, 2u * (uint32_t)k0);
      }
    } else if constexpr (BMODE == B_NT_Q4) {
      st.qc[0] = bload16(rsB0, boff[0], (uint32_t)k0 / 2);
      st.qc[1] = bload16(rsB0, boff[0], (uint32_t)k0 / 2 + 16);
      st.qs[0] = __uint_as_float(bload4(rsB1, boff[1], (uint32_t)k0 / 16));
    } else if constexpr (BMODE == B_NN) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int b = 4 * u + wave;
        const int kr = k0 + 2 * b;            // first of the two rows (even)
        const bool second = kr >= ksplit;     // ksplit is even: no straddle
        uint32_t v = boff[u];
        if (!kfull && kr + (lane >> 5) >= K) v = kOOB;
        dma16(second ? rsB1 : rsB0, Ws + b * 1024, v,
              (uint32_t)((kr - (second ? ksplit : 0)) * p.ldb * 2));
      }
    } else {  // B_NN_Q4: weight rows gk, 8 columns gn.. (4 bytes of codes)
      const int kb = tid >> 5, nb = tid & 31;
      const int gn = n0 + nb * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int gk = k0 + kb * 8 + i;
        const bool ok = gk < K && gn < N;
        const bool first = gk < ksplit;
        const int64_t wr = first ? gk : gk - ksplit;
        const uint8_t *q = (first ? p.Q0 : p.Q1) + wr * (int64_t)(N / 2) + gn / 2;
        const float *sc = (first ? p.S0 : p.S1) + ((wr * (int64_t)N + gn) >> 6);
        const uint32_t cw = *reinterpret_cast<const uint32_t *>(ok ? q : p.Q0);
        const float am = *(ok ? sc : p.S0);
        st.qn[i] = ok ? cw : 0u;
        st.qs[i] = ok ? am : 0.f;
      }
    }
    if constexpr (INLOOP) {
#pragma unroll
      for (int u = 0; u < (RS / 8 + 3) / 4; ++u) {
        const int b = 4 * u + wave;
        if (b < RS / 8) {
          uint32_t v = soff_side[u];
          if (!kfull) {
            const int col = k0 + 8 * (c0 ^ (b & 7));
            if (col >= K) v = kOOB;
          }
          dma16(rsS, Ss + b * 1024, v, 2u * (uint32_t)k0);
        }
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

  // ------------------------------------ register staging -> LDS (non-DMA)
  auto commit_tile = [&](Stage<BMODE> &st, char *stage) {
    char *Ws = stage + XS;
    if constexpr (BMODE == B_NT_Q4) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const u32x4 &src = st.qc[c >> 2];
        lds_write16(Ws, swz_off(tid, c), decode4(src[c & 3], st.qs[0]));
      }
    } else if constexpr (BMODE == B_NN_Q4) {
      const int kb = tid >> 5, nb = tid & 31;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        lds_write16(Ws, nn_off(kb * 8 + i, nb), decode4(st.qn[i], st.qs[i]));
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
  Stage<BMODE> st;
  if (Q4) __syncthreads();  // pair table visible before the first decode
  issue_tile(st, 0, smem);
  commit_tile(st, smem);
  wait_vmem();
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const char *cur = smem + (kt & 1) * STAGE;
    if (kt + 1 < nkt) issue_tile(st, kt + 1, smem + ((kt + 1) & 1) * STAGE);
    {
      // Fragment reads of sub-step kk+1 (and of the side pass during the
      // last sub-step) are in flight while the 16 MFMAs of sub-step kk run;
      // the sched_group_barrier pattern below pins that interleave.
      const char *Xs = cur, *Ws = cur + XS;
      u32x4 fa[2][4], fb[2][4];
      u32x4 sa[2][NSB], xb[2][4];
      auto read_frags = [&](int kk, int bsel) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (NN) {
            const u32x2 lo = lds_read_tr8(Ws, trb[i] + kk * 16 * 512);
            const u32x2 hi = lds_read_tr8(Ws, trb[i] + (kk * 16 + 4) * 512);
            fa[bsel][i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
          } else {
            fa[bsel][i] = lds_read16(Ws, swz_off(wn * 128 + i * 32 + l32, 2 * kk + hi32));
          }
          fb[bsel][i] = lds_read16(Xs, swz_off(wm * 128 + i * 32 + l32, 2 * kk + hi32));
        }
      };
      read_frags(0, 0);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int cb = kk & 1, nb = cb ^ 1;
        if (kk < 3) {
          read_frags(kk + 1, nb);
        } else if constexpr (INLOOP) {
          const char *Ss = cur + XS + WS;
#pragma unroll
          for (int kq = 0; kq < 2; ++kq) {
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb)
              sa[kq][sb] = lds_read16(Ss, swz_off(sb * 16 + l16, 4 * kq + hi16));
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
              xb[kq][mb] = lds_read16(Xs, swz_off(wm * 128 + wn * 64 + mb * 16 + l16, 4 * kq + hi16));
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fa[cb][i], fb[cb][j], acc[i][j]);
      }
      if constexpr (INLOOP) {
#pragma unroll
        for (int kq = 0; kq < 2; ++kq)
#pragma unroll
          for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) sacc[sb][mb] = mfma16(sa[kq][sb], xb[kq][mb], sacc[sb][mb]);
      }
      // schedule: the first sub-step's reads, then per sub-step 16 MFMAs
      // with the next sub-step's reads interleaved one per MFMA
      constexpr int kReads = NN ? 12 : 8;
      constexpr int kSideReads = INLOOP ? 2 * (NSB + 4) : 0;
      sched_group<0x100, kReads>();
#pragma unroll
      for (int kk = 0; kk < 3; ++kk) {
        sched_pairs<kReads>();
        sched_group<0x008, 16 - kReads>();
      }
      sched_pairs<kSideReads>();
      sched_group<0x008, 16 - kSideReads + (INLOOP ? 8 * NSB : 0)>();
    }
    if (kt + 1 < nkt) commit_tile(st, smem + ((kt + 1) & 1) * STAGE);
    wait_vmem();
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
