// bf16 MFMA GEMM with a fused LoRA epilogue, for gfx950.
//
//   C[M x N] = A_op[M x K] . B_op^T  +  S[M x rs] . E[N x rs]^T
//
// S = s * (A_op . SIDE^T) is the rank-r product of the LoRA branch, formed
// once per call by a skinny MFMA kernel ([T x r], bf16) and applied here as a
// second MFMA pass with K = rs in the epilogue ("Unsloth deep-dive", 1.3: the
// layer is the frozen base linear plus x A^T B^T * alpha/r).
//
// This four-wave kernel takes 4-bit weights, decoded while their LDS tiles
// fill (dense bf16 weights go through the eight-wave k_lora_gemm_pp):
//   B_NT_Q4  4-bit codes of an [N x K] weight (forward: W of an nn.Linear,
//            K-contiguous)
//   B_NN_Q4  4-bit codes of the [K x N] weight (backward dX = dY W: W is
//            N-contiguous), decoded into that natural layout in LDS; MFMA
//            fragments are read with the LDS transpose read ds_read_b64_tr_b16
//   B_NT_Q4DQ, B_NN_Q4DQ  the same with double-quantised block constants
//            (8-bit absmax codes decoded through a 256-level table, a scale
//            per 256 blocks and an offset: "Unsloth deep-dive", 1.4)
// The 4-bit decode is bf16_rne(codebook[c] * absmax) with one fp32 multiply
// ("Unsloth code-reading guide", 2.1: 4-bit weights are decoded to bf16
// before every matmul; "Why Unsloth trains 5-8x faster", 5.2: decode fused
// into the matmul).
//
// Epilogues:
//   EPI_STORE       C (bf16), optionally accumulating into C
//   EPI_SWIGLU_FWD  gate/up interleaved tile: e, g, h = silu(e) g (bf16)
//   EPI_SWIGLU_BWD  dh tile: loads saved e, g; writes de, dg (bf16)
//
// Tile 256 x 256, 256 threads = 4 waves in a 2 x 2 grid, each wave a
// 128 x 128 sub-tile of 4 x 4 MFMA 32x32x16 blocks with its 256 fp32
// accumulators in AGPRs.  The MFMA "A" operand is the B_op fragment and the
// "B" operand the A_op fragment, so each lane ends with 4 consecutive output
// columns of one output row (8-byte stores).
//
// Pipeline: token tiles go straight to LDS with buffer_load ... lds; 4-bit
// codes and block constants go to registers one step ahead and are decoded
// into the LDS stage.  K step 64 over 2 stages of 64 KB.  The barrier of each
// step sits before its last 16-K sub-step, so the next stage's first fragment
// reads overlap the current stage's last 16 MFMAs.
#pragma once
#include <type_traits>

#include "common.hpp"

namespace lora {

constexpr int BM = 256, BN = 256, NTHREADS = 256;
// default K step and pipeline depth (template parameters of the kernel;
// the macros exist for tuning sweeps)
#ifndef LORA_GEMM_BK
#define LORA_GEMM_BK 64
#endif
#ifndef LORA_GEMM_NSTAGE
#define LORA_GEMM_NSTAGE 2
#endif
constexpr int kBK = LORA_GEMM_BK, kNSTAGE = LORA_GEMM_NSTAGE;
static_assert(kBK == 32 || kBK == 64, "K step must be 32 or 64");
static_assert(kNSTAGE >= 2 && kNSTAGE <= 4, "2 to 4 pipeline stages");

// 4-bit operand forms of the four-wave kernel (the values 0 and 2 were its
// retired dense forms)
enum BMode { B_NT_Q4 = 1, B_NN_Q4 = 3, B_NT_Q4DQ = 4, B_NN_Q4DQ = 5 };
constexpr bool bmode_nt_q4(int m) { return m == B_NT_Q4 || m == B_NT_Q4DQ; }
constexpr bool bmode_nn_q4(int m) { return m == B_NN_Q4 || m == B_NN_Q4DQ; }
constexpr bool bmode_q4(int m) { return bmode_nt_q4(m) || bmode_nn_q4(m); }
constexpr bool bmode_dq(int m) { return m == B_NT_Q4DQ || m == B_NN_Q4DQ; }
// EPI_SWIGLU_BWD_RANK (eight-wave kernel, rank-r width 16): the SwiGLU'
// epilogue that also forms the tile's shares of the four rank-r products of
// the MLP backward (see GemmArgs::fr_*)
// EPI_STORE_NORM is the store epilogue with per-row factors of a folded
// RMSNorm (rowscale, or nrm_x / nrm_rs / nrm_kk; not both), requested before
// each half of the tile is staged; EPI_SWIGLU_FWD_NORM the SwiGLU forward with
// rowscale, requested before the LoRA pass.  EPI_STORE and EPI_SWIGLU_FWD
// ignore those fields.  (Eight-wave kernel only.)
enum Epi {
  EPI_STORE = 0, EPI_SWIGLU_FWD = 1, EPI_SWIGLU_BWD = 2, EPI_SWIGLU_BWD_RANK = 3,
  EPI_STORE_NORM = 4, EPI_SWIGLU_FWD_NORM = 5
};

struct GemmArgs {
  int M, N, K;
  int ksplit;                   // K index where A0/B0 hand over to A1/B1
  const bf16_t *A0, *A1;        // A_op rows, K-contiguous (A1 after A0 in memory)
  int64_t lda;
  const bf16_t *B0, *B1;        // dense B_op
  int64_t ldb;                  // NT: row stride (>= K); NN: row stride (>= N)
  const uint8_t *Q0, *Q1;       // 4-bit codes
  const float *S0, *S1;         // 4-bit absmax (plain form)
  const float *CB0, *CB1;       // 16 fp32 levels of the Q0 / Q1 weight
  // double-quantised absmax of the Q0 / Q1 weight: 8-bit codes, 256-level
  // tables, one scale per 256 blocks, offsets
  const uint8_t *D0, *D1;
  const float *DT0, *DT1, *DS0, *DS1;
  float doff0, doff1;
  int gu_f;                     // SwiGLU forward: feature count f (N = 2 f)
  const bf16_t *hglob;          // s * (A_op SIDE^T), [M x rs] bf16
  int rs;                       // rank padded to a multiple of 16
  const bf16_t *epi;            // [rows x rs] bf16 epilogue LoRA operand
  // eight-wave SwiGLU forward with rs_seg > 0: when set, the gate rows read
  // epi as Bg [gu_f x rs_seg] and the up rows read epi_u as Bu [gu_f x rs_seg]
  // (the adapters in place, not the interleaved copy)
  const bf16_t *epi_u;
  int accumulate;               // EPI_STORE: C += result
  bf16_t *C;
  int64_t ldc;
  bf16_t *E, *G, *H;            // SwiGLU forward outputs [M x f]; eight-wave
                                // EPI_SWIGLU_BWD: H (optional) gets h = silu(e) g [M x N]
  const bf16_t *Ein, *Gin;      // SwiGLU backward saved activations [M x N]
  bf16_t *DE, *DG;              // SwiGLU backward outputs [M x N], row stride ldd
  int64_t ldd;
  int tiles_m, tiles_n;
  // dense NT store form with N split into up to three segments (fused
  // q/k/v projections): columns [0, nseg1) use B0 / C, [nseg1, nseg2) B1 / C1,
  // [nseg2, N) B2 / C2; boundaries are multiples of the 256-column tile.
  // nseg1 = 0: one segment.
  int nseg1, nseg2;
  // eight-wave kernel: the epilogue operand is block-diagonal with rs_seg
  // columns per block (a multiple of 16).  nseg1 > 0: a tile of segment j
  // runs the LoRA pass over columns [j rs_seg, (j + 1) rs_seg) only; SwiGLU
  // forward: gate rows over block 0, up rows over block 1.  0: all rs columns
  int rs_seg;
  const bf16_t *B2;
  bf16_t *C1, *C2;
  int64_t ldc1, ldc2;
  // RMSNorm folded into the projections that follow it (eight-wave kernel):
  //   rowscale  EPI_SWIGLU_FWD_NORM: e, g of row m are scaled by rowscale[m];
  //             EPI_STORE_NORM: row m of C is (before any accumulation)
  //             (rstd; the GEMM reads the raw rows and weights W diag(w))
  //   cpart     SwiGLU backward: cpart[(tile column * 4 + 64-column block) *
  //             M + m] = sum over the block's columns of de e + dg g
  //             (de, dg as stored); nullptr: not formed
  //   nrm_x     EPI_STORE_NORM: C = nrm_rs[m] acc - nrm_kk[m] nrm_x[m][n] (before any
  //             accumulation), the RMSNorm input gradient; nrm_x is [M x N]
  const float *rowscale;
  float *cpart;
  const bf16_t *nrm_x;
  const float *nrm_rs, *nrm_kk;
  // dense NT (eight-wave, no gate/up interleave): K columns >= kbsplit of the
  // weight operand come from Bk1 (same ldb), kbsplit a multiple of 64;
  // nullptr: one source
  const bf16_t *Bk1;
  int kbsplit;
  // eight-wave NT store form with three K sources for both operands (the
  // fused q/k/v backward's dX read from dQ, dK, dV and Wq^T, Wk^T, Wv^T in
  // place): K columns [mk_kb[j], mk_kb[j + 1]) of the token operand come from
  // mk_a[j] (row stride mk_lda[j]) and of the weight operand from mk_b[j]
  // (row stride mk_ldb[j]); mk_kb[0] = 0, mk_kb[3] = K, every boundary a
  // multiple of the K step (64).  Launched as its own instance; A0, B0, ...
  // are not read then.
  const bf16_t *mk_a[3], *mk_b[3];
  int64_t mk_lda[3], mk_ldb[3];
  int mk_kb[4];
  // EPI_SWIGLU_BWD_RANK: with h = silu(e) g, de, dg as stored, per tile
  //   fr_ud[tn][t][q]       += sum_n h[t][n] Ad[q][n]          (H_d = h Ad^T)
  //   fr_ugu[tn][t][q]      += sum_n de[t][n] Bg[n][q], and at block
  //   fr_ugu[tiles_n + tn]      the same with dg and Bu        ([de Bg | dg Bu])
  //   fr_vd[tm][q][n]       += sum_t G_d[t][q] h[t][n]         (dAd / s)
  //   fr_vgu[tm][q][n], [tm][q][N + n]  sums of H_g[t][q] de[t][n] and
  //                            H_u[t][q] dg[t][n]              (dBg, dBu / s)
  // over the tile's 256 features (tn) or tokens (tm), q < 16, so fixed-order
  // sums over the tiles give the products.  Operands: fr_sd, fr_sg, fr_su
  // [16 x N] bf16 (Ad, Bg^T, Bu^T padded), fr_pd, fr_pg, fr_pu [16 x fr_ldp]
  // bf16 (G_d^T, H_g^T, H_u^T, zero for t >= M; fr_ldp a multiple of 64).
  // EPI_SWIGLU_FWD(_NORM) with fr_ud (else nullptr): with h as stored, per
  // tile of 128 features (tn < tiles_n = ceil(gu_f / 128))
  //   fr_ud[tn][t][q]        = sum over the tile's features n of h[t][n] Ad[q][n]
  // with fr_sd = Ad [16 x gu_f] bf16 (rows >= r zero).
  const bf16_t *fr_sd, *fr_sg, *fr_su, *fr_pd, *fr_pg, *fr_pu;
  int fr_ldp;
  float *fr_ud, *fr_ugu, *fr_vd, *fr_vgu;
};

// XCD-aware, grouped tile order.  Workgroups are dispatched round-robin over
// the 8 XCDs; remapping gives each XCD a contiguous run of logical tiles, and
// the grouped order makes the ~32 tiles resident on one XCD share 4 row
// blocks of A_op and 8 column blocks of B_op in that XCD's L2.
__device__ __forceinline__ void map_tile(int bid, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int nwg = tiles_m * tiles_n;
  int logical = bid;
  if ((nwg & 7) == 0) logical = (bid & 7) * (nwg >> 3) + (bid >> 3);
#ifndef LORA_GEMM_GM
#define LORA_GEMM_GM 4
#endif
  constexpr int GM = LORA_GEMM_GM;
  const int group = logical / (GM * tiles_n);
  const int first_m = group * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int in_group = logical - group * GM * tiles_n;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

// K-contiguous LDS tiles: rows of BK bf16 (BK/8 chunks of 16 bytes), chunk
// index XOR-swizzled so the 16 rows one 16-lane group reads at the same
// logical chunk cover all 64 banks: with 64-byte rows (BK = 32) by
// (row / 4) % 4, with 128-byte rows (BK = 64) by (row / 2) % 8.
template <int BK>
__device__ __forceinline__ uint32_t kc_swz(uint32_t row) {
  return BK == 32 ? ((row >> 2) & 3u) : ((row >> 1) & 7u);
}
template <int BK>
__device__ __forceinline__ uint32_t kc_off(uint32_t row, uint32_t chunk) {
  return row * (2u * BK) + ((chunk ^ kc_swz<BK>(row)) << 4);
}
// NN weight tiles: natural [BK K-rows x 256 N-cols] layout (512-byte rows),
// 16-byte chunk index XORed with 4 (row % 4) so the four rows one 16-lane
// group reads with ds_read_b64_tr_b16 fall in different banks.
__device__ __forceinline__ uint32_t nn_off(uint32_t row, uint32_t chunk) {
  return row * 512u + ((chunk ^ ((row & 3u) << 2)) << 4);
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

template <int BMODE>
struct Stage {  // sized for BK <= 64
  // register-staged 4-bit B operand
  u32x4 qc[2];                           // NT: BK/2 code bytes; NN: 16 per row
  float qs[bmode_nn_q4(BMODE) ? 2 : 1];   // absmax, or the 256-block scale (DQ)
  // NN: bit i = row i comes from the second weight; DQ: bits 8 + i = row i
  // valid, byte i of q8 = row i's 8-bit absmax code
  uint32_t qf;
  uint32_t q8;
};

template <int BMODE, int EPI, int BK = kBK, int NSTAGE = kNSTAGE>
__global__ __launch_bounds__(NTHREADS, 1) void k_lora_gemm(const GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr bool GU = (EPI == EPI_SWIGLU_FWD);
  constexpr bool Q4 = bmode_q4(BMODE);
  static_assert(Q4, "dense weights run in k_lora_gemm_pp");
  constexpr bool DQ = bmode_dq(BMODE);
  constexpr bool NN = bmode_nn_q4(BMODE);
  constexpr int XS = BM * BK * 2, WS = BN * BK * 2;
  constexpr int STAGE = XS + WS;
  constexpr int kReads = NN ? 12 : 8;   // LDS reads per 16-K sub-step
  constexpr int KSUB = BK / 16;          // 16-K MFMA sub-steps per K step
  constexpr int RPI = 1024 / (2 * BK);   // tile rows per 1-KB DMA instruction
  constexpr int NDMA = BM / RPI / 4;     // DMA instructions per wave per operand tile
  constexpr int CPR = BK / 8;            // 16-byte chunks per row
  static_assert(NSTAGE >= 2 && NSTAGE <= 5, "pipeline depth");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi32 = lane >> 5;

  int tm, tn;
  map_tile(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K, ksplit = p.ksplit;

  // 4-bit pair tables of the Q0 and Q1 weights, then (DQ) their 256-level
  // absmax tables
  float2 *cbt = reinterpret_cast<float2 *>(smem + NSTAGE * STAGE);
  float *dqt = reinterpret_cast<float *>(smem + NSTAGE * STAGE + 4096);
  if constexpr (Q4) {
    // entry b = (codebook[b & 15], codebook[b >> 4]): a code byte decodes
    // into its two elements with one LDS read
    cbt[tid] = make_float2(p.CB0[tid & 15], p.CB0[tid >> 4]);
    cbt[256 + tid] = make_float2(p.CB1[tid & 15], p.CB1[tid >> 4]);
    if constexpr (DQ) {
      dqt[tid] = p.DT0[tid];
      dqt[256 + tid] = p.DT1[tid];
    }
  }

  // ---------------------------------------------------- DMA lane geometry
  // A tile: DMA instruction u of wave w fills rows RPI b .. RPI b + RPI-1
  // (b = 4u + w); lane l lands in row RPI b + l/CPR at chunk l%CPR, which
  // holds logical chunk c = (l%CPR) ^ swz(row).
  auto dma_row = [&](int u) { return RPI * (4 * u + wave) + lane / CPR; };
  auto dma_chunk = [&](int u) { return (lane % CPR) ^ (int)kc_swz<BK>(dma_row(u)); };
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(p.A0 + (int64_t)m0 * p.lda, kMaxRecords);
  // A1 - A0 - 2 ksplit: added to offsets of columns >= ksplit
  const uint32_t dA1 = (uint32_t)((const char *)p.A1 - (const char *)p.A0) - 2u * (uint32_t)ksplit;
  uint32_t aoff[NDMA];
#pragma unroll
  for (int u = 0; u < NDMA; ++u) {
    const int row = dma_row(u);
    aoff[u] = (m0 + row < M) ? (uint32_t)(row * p.lda * 2 + dma_chunk(u) * 16) : kOOB;
  }
  uint32_t boff[2];
  __amdgpu_buffer_rsrc_t rsB0, rsB1;
  if constexpr (bmode_nt_q4(BMODE)) {
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
    rsB0 = make_rsrc((up ? p.Q1 : p.Q0) + grow0 * (K / 2), kMaxRecords);
    rsB1 = make_rsrc((up ? p.S1 : p.S0) + grow0 * (K / 64), kMaxRecords);
    const bool ok = GU ? (jg < p.gu_f) : (jg < N);
    boff[0] = ok ? (uint32_t)(jl * (K / 2)) : kOOB;       // codes
    boff[1] = ok ? (uint32_t)(jl * (K / 64) * 4) : kOOB;  // absmax
    if constexpr (DQ) {
      // flat index of the row's first 64-block in its own weight; -1: the
      // row lies outside the weight
      boff[1] = ok ? (uint32_t)((grow0 + jl) * (K / 64)) : 0xFFFFFFFFu;
    }
  }
  // NT 4-bit: this thread's tables (gate or up weight)
  const int tsel = (bmode_nt_q4(BMODE) && GU && ((tid >> 6) & 1)) ? 256 : 0;
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

  const int nkt = (K + BK - 1) / BK;
  // ---------------------------------------- DMA of K step kt into a stage
  // Steps past the end issue loads whose lanes are all out of range (they
  // write zeros into a stage nobody reads), which keeps the per-wave count
  // of outstanding loads uniform for the vmcnt waits.
  auto issue_dma = [&](int kt, char *stage) {
    const int k0 = kt * BK;
    char *Xs = stage;
    const bool live = kt < nkt;
    const bool full = live && (k0 + BK <= K) && (k0 + BK <= ksplit || k0 >= ksplit);
    if (full) {
      const uint32_t sa = 2u * (uint32_t)k0 + (k0 >= ksplit ? dA1 : 0u);
#pragma unroll
      for (int u = 0; u < NDMA; ++u) dma16(rsA, Xs + (4 * u + wave) * 1024, aoff[u], sa);
    } else {
#pragma unroll
      for (int u = 0; u < NDMA; ++u) {
        const int col = k0 + 8 * dma_chunk(u);
        const uint32_t v = (live && aoff[u] != kOOB && col < K)
                               ? aoff[u] + 2u * (uint32_t)k0 + (col >= ksplit ? dA1 : 0u)
                               : kOOB;
        dma16(rsA, Xs + (4 * u + wave) * 1024, v, 0);
      }
    }
  };

  // ----------------------------- 4-bit weights: global -> registers -> LDS
  auto load_q4 = [&](Stage<BMODE> &st, int kt) {
    const int k0 = kt * BK;
    const bool live = kt < nkt;
    if constexpr (bmode_nt_q4(BMODE)) {
      // BK codes (BK/2 bytes) and the row's absmax of this K step
#pragma unroll
      for (int h = 0; h < BK / 32; ++h)
        st.qc[h] = bload16(rsB0, live ? boff[0] : kOOB, (uint32_t)k0 / 2 + 16 * h);
      if constexpr (DQ) {
        // the block's 8-bit code and its 256-block scale (index 0 stands
        // in for rows outside the weight; commit zeroes their absmax)
        const bool ok = live && boff[1] != 0xFFFFFFFFu;
        const uint32_t b = ok ? boff[1] + (uint32_t)(k0 / 64) : 0u;
        const bool up = tsel != 0;
        st.q8 = (up ? p.D1 : p.D0)[b];
        st.qs[0] = (up ? p.DS1 : p.DS0)[b >> 8];
        st.qf = ok ? 0x100u : 0u;
      } else {
        st.qs[0] = __uint_as_float(bload4(rsB1, live ? boff[1] : kOOB, (uint32_t)(k0 / 64) * 4));
      }
    } else if constexpr (bmode_nn_q4(BMODE)) {
      // weight rows k0 + kr + 32 i (i < BK/32), 32 columns gn .. gn+31 each:
      // 16 code bytes (one 16-byte load) and one absmax, since N % 64 == 0
      // puts the 32 columns inside one 64-block
      const int kr = tid >> 3, gn = n0 + 32 * (tid & 7);
      st.qf = 0u;
      if constexpr (DQ) st.q8 = 0u;
#pragma unroll
      for (int i = 0; i < BK / 32; ++i) {
        const int gk = k0 + kr + 32 * i;
        const bool ok = live && gk < K && gn < N;
        const bool first = gk < ksplit;
        const int64_t wr = first ? gk : gk - ksplit;
        const int64_t e0 = wr * (int64_t)N + gn;   // flat element index in its weight
        const uint8_t *q = (first ? p.Q0 : p.Q1) + e0 / 2;
        const int64_t blk = e0 >> 6;
        const u32x4 cv = gload16(ok ? q : p.Q0);
        st.qc[i] = cv;
        if (!ok) st.qc[i] = u32x4{0u, 0u, 0u, 0u};
        st.qf |= (first ? 0u : 1u) << i;
        if constexpr (DQ) {
          const int64_t b = ok ? blk : 0;
          const uint32_t c8 = (first ? p.D0 : p.D1)[b];
          st.qs[i] = (first ? p.DS0 : p.DS1)[b >> 8];
          st.q8 |= (ok ? c8 : 0u) << (8 * i);
          st.qf |= (ok ? 1u : 0u) << (8 + i);
        } else {
          const float *sc = (first ? p.S0 : p.S1) + blk;
          const float am = *(ok ? sc : p.S0);
          st.qs[i] = ok ? am : 0.f;
        }
      }
    }
  };
  // DQ: absmax of a staged block from its 8-bit code and scale (second
  // weight's tables when `second`); 0 for blocks outside the weight
  auto dq_absmax = [&](uint32_t c8, float scale, bool second, bool valid) -> float {
    const float am = absmax_dq(dqt[(second ? 256 : 0) + c8], scale, second ? p.doff1 : p.doff0);
    return valid ? am : 0.f;
  };
  // 4 code bytes (8 elements) -> 8 bf16 packed in 4 words
  auto decode4 = [&](uint32_t cw, float am, int tb) -> u32x4 {
    u32x4 o;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float2 cv = cbt[tb + ((cw >> (8 * b)) & 0xFFu)];
      o[b] = pack_bf16x2(cv.x * am, cv.y * am);
    }
    return o;
  };
  auto commit_q4 = [&](Stage<BMODE> &st, char *stage) {
    char *Ws = stage + XS;
    if constexpr (bmode_nt_q4(BMODE)) {
      float am = st.qs[0];
      if constexpr (DQ) am = dq_absmax(st.q8, st.qs[0], tsel != 0, st.qf != 0u);
#pragma unroll
      for (int c = 0; c < CPR; ++c)
        lds_write16(Ws, kc_off<BK>(tid, c), decode4(st.qc[c >> 2][c & 3], am, tsel));
    } else if constexpr (bmode_nn_q4(BMODE)) {
      // row kr + 32 i, chunks 4 cg .. 4 cg + 3.  Lanes with cg >= 4 write
      // their chunks rotated by one, so the 8 lanes of one row (64-byte
      // slots, cg and cg + 4 a bank period apart) hit distinct banks.
      const int kr = tid >> 3, cg = tid & 7, rot = cg >> 2;
#pragma unroll
      for (int i = 0; i < BK / 32; ++i) {
        const bool second = (st.qf >> i) & 1u;
        float am = st.qs[i];
        if constexpr (DQ)
          am = dq_absmax((st.q8 >> (8 * i)) & 0xFFu, st.qs[i], second, (st.qf >> (8 + i)) & 1u);
        const u32x4 c = st.qc[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // word (j + rot) & 3 by selects (an indexed vector read would go
          // through scratch memory)
          const uint32_t w = rot ? c[(j + 1) & 3] : c[j];
          lds_write16(Ws, nn_off(kr + 32 * i, 4 * cg + ((j + rot) & 3)),
                      decode4(w, am, second ? 256 : 0));
        }
      }
    }
  };

  // ---------------------------------------------------- fragment reads
  u32x4 fa[2][4], fb[2][4];
  auto read_frags = [&](const char *stage, int kk, int bsel) {
    const char *Xs = stage, *Ws = stage + XS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (NN) {
        const u32x2 lo = lds_read_tr8(Ws, trb[i] + kk * 16 * 512);
        const u32x2 hi = lds_read_tr8(Ws, trb[i] + (kk * 16 + 4) * 512);
        fa[bsel][i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      } else {
        fa[bsel][i] = lds_read16(Ws, kc_off<BK>(wn * 128 + i * 32 + l32, 2 * kk + hi32));
      }
      fb[bsel][i] = lds_read16(Xs, kc_off<BK>(wm * 128 + i * 32 + l32, 2 * kk + hi32));
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  auto mfmas = [&](int bsel) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fa[bsel][i], fb[bsel][j], acc[i][j]);
  };

  // ---------------------------------------------------------- prologue
  Stage<BMODE> st;
  __syncthreads();  // pair table visible before the first decode
  load_q4(st, 0);
#pragma unroll
  for (int i = 0; i < NSTAGE - 1; ++i) issue_dma(i, smem + i * STAGE);
  wait_vmem();
  commit_q4(st, smem);
  __syncthreads();
  read_frags(smem, 0, 0);

  // ------------------------------------------------------------ K loop
  // A wave's loads, oldest first, when it reaches the wait before the
  // step's barrier: DMA(kt+1) .. DMA(kt+NSTAGE-2), q4(kt+1), DMA(kt+NSTAGE-1).
  // Waiting until only the youngest DMA step remains completes DMA(kt+1)
  // and the 4-bit registers of step kt+1.  The barrier sits before the
  // step's last 16-K sub-step, whose MFMAs overlap the next stage's first
  // fragment reads.
  constexpr int kWaitQ4 = NSTAGE == 2 ? 0 : NDMA;
  auto step = [&](int kt) {
    const char *cur = smem + (kt % NSTAGE) * STAGE;
    char *nxt = smem + ((kt + 1) % NSTAGE) * STAGE;
    char *tgt = smem + ((kt + NSTAGE - 1) % NSTAGE) * STAGE;
    load_q4(st, kt + 1);
    issue_dma(kt + NSTAGE - 1, tgt);
#pragma unroll
    for (int kk = 0; kk + 1 < KSUB; ++kk) {
      // sub-step kk: MFMAs on fragment set kk&1, reads of kk+1 interleaved
      read_frags(cur, kk + 1, (kk + 1) & 1);
      mfmas(kk & 1);
      sched_pairs<kReads>();
      sched_group<0x008, 16 - kReads>();
    }
    // keep every MFMA of the earlier sub-steps ahead of the wait: the
    // longer the loads have, the less the wait stalls
    __builtin_amdgcn_sched_barrier(0);
    vm_wait<kWaitQ4>();
    commit_q4(st, nxt);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier_only();
    __builtin_amdgcn_sched_barrier(0);
    // last sub-step: MFMAs on its fragment set, the next stage's first
    // reads interleaved (on the last step they read a stage nobody uses)
    read_frags(nxt, 0, 0);
    mfmas((KSUB - 1) & 1);
    sched_pairs<kReads>();
    sched_group<0x008, 16 - kReads>();
  };
  for (int kt = 0; kt < nkt; ++kt) step(kt);
  wait_vmem();

  // ------------------------------------------------ LoRA epilogue pass
  // acc += S . E^T with K = rs: S = s (A_op SIDE^T) [M x rs], E [N x rs]
  const int rs = p.rs;
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
      const int m = m0 + wm * 128 + j * 32 + l32;
      u32x4 v = {0, 0, 0, 0};
      if (m < M) v = gload16(p.hglob + (int64_t)m * rs + kq * 16 + 8 * hi32);
      hb[j] = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(ea[i], hb[j], acc[i][j]);
  }

  // ------------------------------------------------ output
  // The accumulators hold 4 consecutive output columns of one token row per
  // lane, 32 rows per instruction: stored directly that would scatter 8-byte
  // pieces over 32 rows.  Each wave instead passes its 128 x 128 sub-tile
  // through a private 32 KB LDS region, 64 token rows (fp32) at a time, and
  // then reads and writes global memory in 16-byte pieces along rows (a
  // wave instruction covers whole 128- or 256-byte row segments).
  // Region layout: row r (0..63) of 512 bytes, 16-byte chunk c (4 columns)
  // stored at chunk c ^ (r % 32), so the 16 rows one write instruction
  // touches land in distinct banks.
  __syncthreads();   // every wave is done with the pipeline stages
  char *reg = smem + wave * 32768;
  auto ep_off = [](int r, int c) -> uint32_t { return (uint32_t)(r * 512 + ((c ^ (r & 31)) << 4)); };
  // SwiGLU backward: a half's saved e, g (16 row groups x 16 bytes each per
  // lane) are all requested before the half is staged, so their latency is
  // paid once per half
  u32x4 ein[16], gin[16];
  auto load_eg = [&](int half) {
    if constexpr (EPI == EPI_SWIGLU_BWD) {
      const int q = lane & 15, n = n0 + wn * 128 + 8 * q;
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int m = m0 + wm * 128 + half * 64 + it * 4 + (lane >> 4);
        u32x4 e = {0, 0, 0, 0}, g = {0, 0, 0, 0};
        if (m < M && n < N) {
          const int64_t off = (int64_t)m * N + n;
          e = gload16(p.Ein + off);
          g = gload16(p.Gin + off);
        }
        ein[it] = e;
        gin[it] = g;
      }
    }
  };
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    load_eg(half);
    // rows (j - 2 half) * 32 + l32 of the region hold acc[.][j]
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int j = 2 * half + jj;
          const f32x16 &a = acc[i][j];
          const u32x4 v = {__float_as_uint(a[4 * g]), __float_as_uint(a[4 * g + 1]),
                           __float_as_uint(a[4 * g + 2]), __float_as_uint(a[4 * g + 3])};
          lds_write16(reg, ep_off(jj * 32 + l32, 8 * i + 2 * g + hi32), v);
        }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    const int mrow0 = m0 + wm * 128 + half * 64;   // token of region row 0
    if constexpr (EPI == EPI_SWIGLU_FWD) {
      // region columns 0..63: gate, 64..127: up (features tn*128 + wn*64 + c)
      const int f = p.gu_f;
      const int q = lane & 7;                       // 8-column group
#pragma unroll 2
      for (int it = 0; it < 8; ++it) {
        const int r = it * 8 + (lane >> 3);
        const int m = mrow0 + r;
        const int jf = tn * 128 + wn * 64 + 8 * q;
        const u32x4 e0 = lds_read16(reg, ep_off(r, 2 * q)), e1 = lds_read16(reg, ep_off(r, 2 * q + 1));
        const u32x4 g0 = lds_read16(reg, ep_off(r, 16 + 2 * q)), g1 = lds_read16(reg, ep_off(r, 17 + 2 * q));
        if (m < M && jf < f) {
          const float ev[8] = {__uint_as_float(e0[0]), __uint_as_float(e0[1]), __uint_as_float(e0[2]),
                               __uint_as_float(e0[3]), __uint_as_float(e1[0]), __uint_as_float(e1[1]),
                               __uint_as_float(e1[2]), __uint_as_float(e1[3])};
          const float gv[8] = {__uint_as_float(g0[0]), __uint_as_float(g0[1]), __uint_as_float(g0[2]),
                               __uint_as_float(g0[3]), __uint_as_float(g1[0]), __uint_as_float(g1[1]),
                               __uint_as_float(g1[2]), __uint_as_float(g1[3])};
          u32x4 ew, gw, hw;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            ew[t] = pack_bf16x2(ev[2 * t], ev[2 * t + 1]);
            gw[t] = pack_bf16x2(gv[2 * t], gv[2 * t + 1]);
            // h from the rounded e, g: the same values the backward reloads
            const float ea = bf16lo(ew[t]), eb = bf16hi(ew[t]);
            const float ga = bf16lo(gw[t]), gb = bf16hi(gw[t]);
            hw[t] = pack_bf16x2(ea * sigmoidf_fast(ea) * ga, eb * sigmoidf_fast(eb) * gb);
          }
          const int64_t off = (int64_t)m * f + jf;
          gstore16(p.E + off, ew);
          gstore16(p.G + off, gw);
          gstore16(p.H + off, hw);
        }
      }
    } else {
      const int q = lane & 15;                      // 8-column group
      const int n = n0 + wn * 128 + 8 * q;
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int r = it * 4 + (lane >> 4);
        const int m = mrow0 + r;
        const u32x4 a0 = lds_read16(reg, ep_off(r, 2 * q)), a1 = lds_read16(reg, ep_off(r, 2 * q + 1));
        if (m >= M || n >= N) continue;
        float v[8] = {__uint_as_float(a0[0]), __uint_as_float(a0[1]), __uint_as_float(a0[2]),
                      __uint_as_float(a0[3]), __uint_as_float(a1[0]), __uint_as_float(a1[1]),
                      __uint_as_float(a1[2]), __uint_as_float(a1[3])};
        if constexpr (EPI == EPI_STORE) {
          bf16_t *cb = p.C;
          int64_t ldc = p.ldc;
          int ncs = 0;
          if (p.nseg1 > 0 && n0 >= p.nseg1) {
            const bool s2 = p.nseg2 > 0 && n0 >= p.nseg2;
            cb = s2 ? p.C2 : p.C1;
            ldc = s2 ? p.ldc2 : p.ldc1;
            ncs = s2 ? p.nseg2 : p.nseg1;
          }
          bf16_t *dst = cb + (int64_t)m * ldc + (n - ncs);
          if (p.accumulate) {
            const u32x4 o = gload16(dst);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              v[2 * t] += bf16lo(o[t]);
              v[2 * t + 1] += bf16hi(o[t]);
            }
          }
          u32x4 w;
#pragma unroll
          for (int t = 0; t < 4; ++t) w[t] = pack_bf16x2(v[2 * t], v[2 * t + 1]);
          gstore16(dst, w);
        } else {  // EPI_SWIGLU_BWD: v = dh
          const int64_t off = (int64_t)m * N + n;
          const u32x4 ev = ein[it], gv = gin[it];
          u32x4 dew, dgw;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            float de[2], dg[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const float e = h2 ? bf16hi(ev[t]) : bf16lo(ev[t]);
              const float gg = h2 ? bf16hi(gv[t]) : bf16lo(gv[t]);
              const float dh = v[2 * t + h2];
              const float sg = sigmoidf_fast(e);
              dg[h2] = dh * e * sg;
              de[h2] = dh * gg * sg * (1.0f + e * (1.0f - sg));
            }
            dew[t] = pack_bf16x2(de[0], de[1]);
            dgw[t] = pack_bf16x2(dg[0], dg[1]);
          }
          const int64_t doff = (int64_t)m * p.ldd + n;
          gstore16(p.DE + doff, dew);
          gstore16(p.DG + doff, dgw);
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
  }
}

template <int BMODE, int BK = kBK, int NSTAGE = kNSTAGE>
constexpr size_t gemm_lds_bytes() {
  // pipeline stages (at least the 4 x 32 KB the output staging uses), then
  // the two weights' 4-bit pair tables and (double-quantised) 256-level
  // block-constant tables
  return (NSTAGE * (BM * BK * 2 + BN * BK * 2) > 4 * 32768 ? (size_t)NSTAGE * (BM * BK * 2 + BN * BK * 2)
                                                           : (size_t)4 * 32768) +
         2 * 256 * sizeof(float2) + (bmode_dq(BMODE) ? 2 * 256 * sizeof(float) : 0);
}

}  // namespace lora
