// Eight-wave ("ping-pong") dense LoRA GEMM for gfx950: every bf16-weight
// product of the library.
//
// Contract as documented at GemmArgs (256 x 256 output tile;
// K = rs LoRA epilogue pass adding S . E^T, "Unsloth deep-dive" 1.3; store,
// SwiGLU and SwiGLU' epilogues), run by 512 threads: two waves per SIMD, in
// two groups of four (waves 0-3 and 4-7, one of each on every SIMD).  The
// groups alternate between
//   a compute phase: 32 back-to-back MFMA 32x32x16 on one K step (64) of
//     fragments already in registers, and
//   a memory phase: the LDS fragment reads of its next K step and the
//     LDS-DMA of one operand tile of a later K step (group 0: tokens,
//     group 1: weights),
// with a workgroup barrier between phases, so that while one wave of a SIMD
// waits on its vector-memory issue the other keeps the matrix core busy.
// With one wave per SIMD (the four-wave form) those stalls sit between the
// wave's own MFMAs.  Each wave owns a 128 (tokens) x 64 (weight rows)
// sub-tile: 128 fp32 accumulators per lane, 96 registers of fragments.
//
// Phase schedule (token tile of step s in LDS stage s % 2, weight tile in
// stage s % 3):
//   G0: read s=0 | C0 | M1 | C1 | M2 ...   Ms: read s, load token tile s+1
//                                          (store form: load, then read)
//   G1:   --     | M0 | C0 | M1 | C1 ...   Ms: load weight tile s+2, read s
// Every load targets a stage whose last reads ended before an earlier
// barrier, and each group drains all of its loads (vmcnt 0) before the
// barrier that precedes their first read, with no younger load in flight.
//
// Gate/up tiles (SwiGLU forward) interleave weight rows in 32-row blocks,
// [32 gate | 32 up] per 64 tile rows, so every wave's 64 columns hold the
// gate and up values of the same 32 features.
//
// NN = true: the weight operand is W as stored, [K x N] with N contiguous
// (backward dX = dY W without a transposed copy).  Its LDS tile keeps that
// layout, [64 K-rows x 256 columns], and the MFMA fragments are read with
// the LDS transpose read ds_read_b64_tr_b16 (two per 32-column block and
// 16-K sub-step).  K rows >= ksplit come from the second weight (B1).  The
// NN form keeps two stages of both tiles, every wave loading a share of
// each (group 1 a quarter, inside its compute phase): with the weight tile loaded by
// group 1 alone it ran 6-13 % slower than this, while the NT forms run up to
// 5 % faster with the split loads.

#pragma once
#include "gemm_lora.hpp"

namespace lora {

constexpr int PP_THREADS = 512;
// NT: two 32 KB stages of the token tile and three of the weight tile (K
// step 64); NN: two stages of both.  The epilogue reuses the first 128 KB
// (8 x 16 KB).
constexpr size_t pp_lds(bool nn) { return (nn ? 4 : 5) * (size_t)32768; }

__device__ __forceinline__ void pp_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int EPI, bool NN = false, bool MK = false>
__global__ __launch_bounds__(PP_THREADS, 1) void k_lora_gemm_pp(const GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr bool GU = (EPI == EPI_SWIGLU_FWD || EPI == EPI_SWIGLU_FWD_NORM);
  static_assert(!(NN && GU), "the gate/up forward reads its weights K-contiguous");
  static_assert(!MK || (EPI == EPI_STORE && !NN), "three K sources: the NT store form only");
  constexpr int BK = 64, XS = BM * BK * 2, WS = BN * BK * 2;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int wm = wave & 1, wn = wave >> 1;   // token half, 64-row weight quarter
  const int l32 = lane & 31, hi32 = lane >> 5;

  int tm, tn;
  map_tile(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K, ksplit = p.ksplit;

  u32x4 fw[4][2], ft[4][4];   // [16-K sub-step][32-row block]: weight rows, tokens
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  auto comp = [&]() {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fw[kk][i], ft[kk][j], acc[i][j]);
    // the phase's MFMAs stay ahead of its closing wait and barrier
    __builtin_amdgcn_sched_barrier(0);
  };
  auto lgkm0 = []() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };
  if constexpr (NN) {
    // ------------------------------------------ NN form: shared loads
    // Two stages of both tiles.  Each of a K step's 32 token blocks (rows
    // 8b .. 8b+7) and 32 weight blocks (K rows 2b, 2b+1) is loaded by one
    // wave: group-0 wave w blocks w + 4u (u < 6) of both tiles, in its
    // memory phase, into the stage both groups finished reading before the
    // barrier that opened it; group-1 wave w blocks 24 + w + 4u (u < 2),
    // inside its compute phase, one load after every two of its first MFMAs,
    // i.e. after the barrier that closed every read of that stage (measured
    // 1-2 % faster than an even 8 / 8 share).  Group 0 drains its loads at
    // the end of its next compute phase, group 1 at the end of its next
    // memory phase.  Token block b = b0 + 4u holds rows r0 + 32u
    // (r0 = 8 b0 + l/8); its swizzled chunk does not depend on u.
    constexpr int NI0 = 6, NI1 = 2;
    const int b0 = grp ? 4 * NI0 + (wave & 3) : (wave & 3);
    const int r0 = 8 * b0 + (lane >> 3);
    const int cA = (lane & 7) ^ (int)kc_swz<BK>(r0);
    const int kcol = 8 * cA;
    const __amdgpu_buffer_rsrc_t rsA = make_rsrc(p.A0 + (int64_t)m0 * p.lda, kMaxRecords);
    const uint32_t dA1 = (uint32_t)((const char *)p.A1 - (const char *)p.A0) - 2u * (uint32_t)ksplit;
    const uint32_t aoff0 = (uint32_t)(r0 * p.lda * 2 + cA * 16);
    const uint32_t astep = (uint32_t)(32 * p.lda * 2);   // 32 tile rows
    const int arem = M - m0 - r0;
    // weight K rows 2b, 2b+1: lane l lands in row 2b + l/32 at physical
    // chunk l%32, holding columns 8c .. 8c+7 with c = (l%32) ^ 4 (row%4);
    // row%4 does not depend on u
    const int krow = 2 * b0 + (lane >> 5);
    const int cn = (lane & 31) ^ ((krow & 3) << 2);
    // The weight descriptors are rebased on every K step (row k0 of the
    // step, in each source's own row numbering), so every offset stays
    // inside one step's 64 rows whatever the weight's size.  A row kr >= ksplit
    // of a step that starts in the first source sits at (kr - k0) rows from
    // the second source's base for that step, as it does in the first.
    const int64_t ldb2 = 2 * p.ldb;
    const char *const wbase0 = (const char *)(p.B0 + n0);
    const char *const wbase1 = (const char *)(p.B1 + n0) - (int64_t)ksplit * ldb2;
    const uint32_t boff0 = (n0 + 8 * cn < N) ? (uint32_t)((lane >> 5) * ldb2 + cn * 16) : kOOB;
    const int nk = (K + BK - 1) / BK;
    constexpr int STAGE = XS + WS;
    auto dma = [&](auto ni_tag, int kt, int stg) {
      constexpr int NI = decltype(ni_tag)::value;
      char *Xs = smem + stg * STAGE, *Ws = Xs + XS;
      const int k0 = kt * BK;
      const int col = k0 + kcol;
      const bool kin = col < K;
      const uint32_t ka = 2u * (uint32_t)k0 + (col >= ksplit ? dA1 : 0u);
#pragma unroll
      for (int u = 0; u < NI; ++u) {
        const bool ok = kin && 32 * u < arem;
        dma16(rsA, Xs + (b0 + 4 * u) * 1024, ok ? aoff0 + (uint32_t)u * astep + ka : kOOB, 0);
      }
      const __amdgpu_buffer_rsrc_t rsB = make_rsrc(wbase0 + (int64_t)k0 * ldb2, kMaxRecords);
      const __amdgpu_buffer_rsrc_t rsB1 = make_rsrc(wbase1 + (int64_t)k0 * ldb2, kMaxRecords);
#pragma unroll
      for (int u = 0; u < NI; ++u) {
        const int b = b0 + 4 * u;
        const int kr = k0 + 2 * b;          // first of the two K rows (even)
        const bool second = kr >= ksplit;   // ksplit is even: no straddle
        const bool ok = kr + (lane >> 5) < K;
        dma16(second ? rsB1 : rsB, Ws + b * 1024, ok ? boff0 : kOOB, (uint32_t)(2 * b * ldb2));
      }
    };
    // byte offset of this lane's transpose-read row for column block i at K
    // sub-step 0 (rows kk*16 and kk*16 + 4 are reached with immediates)
    uint32_t trb[2];
    {
      const int g = lane >> 4, sl = lane & 15;
      const int krow0 = 8 * (g >> 1) + (sl >> 2);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int nl = wn * 64 + i * 32 + 16 * (g & 1) + 4 * (sl & 3);
        trb[i] = nn_off(krow0, nl >> 3) + ((nl >> 2) & 1) * 8;
      }
    }
    auto rd = [&](int stg) {
      const char *Xs = smem + stg * STAGE, *Ws = Xs + XS;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const u32x2 lo = lds_read_tr8(Ws, trb[i] + kk * 16 * 512);
          const u32x2 hi = lds_read_tr8(Ws, trb[i] + (kk * 16 + 4) * 512);
          fw[kk][i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          ft[kk][j] = lds_read16(Xs, kc_off<BK>(wm * 128 + j * 32 + l32, 2 * kk + hi32));
      }
    };
    using G0N = std::integral_constant<int, NI0>;
    using G1N = std::integral_constant<int, NI1>;
    auto comp_dma = [&](int kt, int stg) {
      dma(G1N{}, kt, stg);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fw[kk][i], ft[kk][j], acc[i][j]);
#pragma unroll
      for (int i = 0; i < 2 * NI1; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 32 - 4 * NI1, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    if (grp == 0) {
      dma(G0N{}, 0, 0);
      if (nk > 1) dma(G0N{}, 1, 1);
    } else {
      dma(G1N{}, 0, 0);
      if (nk > 1) dma(G1N{}, 1, 1);
    }
    wait_vmem();
    pp_barrier();
    if (grp == 0) {
      rd(0);
      lgkm0();
      pp_barrier();
      for (int s = 0; s < nk; ++s) {
        comp();              // step s
        wait_vmem();         // own share of step s+1 (issued one phase ago)
        pp_barrier();
        if (s + 1 < nk) rd((s + 1) & 1);
        if (s + 2 < nk) dma(G0N{}, s + 2, s & 1);
        lgkm0();
        pp_barrier();
      }
    } else {
      pp_barrier();
      int s = 0;
      for (; s + 2 < nk; ++s) {
        rd(s & 1);
        lgkm0();
        wait_vmem();         // own share of step s+1 (issued one phase ago)
        pp_barrier();
        comp_dma(s + 2, s & 1);   // step s
        pp_barrier();
      }
      for (; s < nk; ++s) {
        rd(s & 1);
        lgkm0();
        wait_vmem();
        pp_barrier();
        comp();
        pp_barrier();
      }
    }
  } else {
    // ---------------------------------------------------- DMA lane geometry
    // LDS: two stages of the A_op tile (tokens, 32 KB each) and three of the
    // B_op tile (weights, 32 KB each), 160 KB.  Group 0 loads every A tile,
    // group 1 every B tile, each in its memory phase and each into a stage that
    // every wave finished reading before an earlier barrier (see the K loop).
    // A tile of 32 one-kilobyte blocks, block b = rows 8b .. 8b+7: wave w of a
    // group issues blocks w + 4u (u < 8); lane l lands in row r0 + 32u
    // (r0 = 8w + l/8) at physical chunk l%8, which holds logical chunk
    // c = (l%8) ^ swz(row), i.e. K columns 8c .. 8c+7.  swz(row) = (row/2) % 8
    // does not depend on u, so neither does c.  B tiles: the same geometry
    // (dense NT), or two K rows per block (NN).
    constexpr int NI = 8;
    constexpr int ASTG = 2, BSTG = 3;
    const int w4 = wave & 3;
    const int r0 = 8 * w4 + (lane >> 3);
    const int cA = (lane & 7) ^ (int)kc_swz<BK>(r0);
    const int kcol = 8 * cA;
    char *const a_lds = smem;                       // A stage i at a_lds + i * XS
    char *const b_lds = smem + ASTG * XS;           // B stage i at b_lds + i * WS
    const __amdgpu_buffer_rsrc_t rsA = make_rsrc(p.A0 + (int64_t)m0 * p.lda, kMaxRecords);
    // A1 - A0 - 2 ksplit: added to offsets of columns >= ksplit
    const uint32_t dA1 = (uint32_t)((const char *)p.A1 - (const char *)p.A0) - 2u * (uint32_t)ksplit;
    const uint32_t aoff0 = (uint32_t)(r0 * p.lda * 2 + cA * 16);
    const uint32_t astep = (uint32_t)(32 * p.lda * 2);   // 32 tile rows
    const int arem = M - m0 - r0;                         // block u valid if 32u < arem
    __amdgpu_buffer_rsrc_t rsB, rsB1;
    uint32_t boff0;
    int brem;
    if constexpr (GU) {
      // tile row r0 + 32u: feature 32 (u / 2) + r0 of the tile, of the gate
      // weight for even u and of the up weight for odd u
      rsB = make_rsrc(p.B0 + (int64_t)tn * 128 * p.ldb, kMaxRecords);
      rsB1 = make_rsrc(p.B1 + (int64_t)tn * 128 * p.ldb, kMaxRecords);
      boff0 = (uint32_t)(r0 * p.ldb * 2 + cA * 16);
      brem = p.gu_f - tn * 128 - r0;
    } else {
      const bf16_t *bseg = p.B0;
      int nsb = 0;
      if (p.nseg1 > 0 && n0 >= p.nseg1) {
        const bool s2 = p.nseg2 > 0 && n0 >= p.nseg2;
        bseg = s2 ? p.B2 : p.B1;
        nsb = s2 ? p.nseg2 : p.nseg1;
      }
      rsB = rsB1 = make_rsrc(bseg + (int64_t)(n0 - nsb) * p.ldb, kMaxRecords);
      boff0 = (uint32_t)(r0 * p.ldb * 2 + cA * 16);
      brem = N - n0 - r0;
    }
    // a second K source for K columns >= kbsplit (a multiple of the K step):
    // its base is shifted back by kbsplit columns, so a step's offsets are
    // the same expression for either source and only the base changes
    const char *const bk1base =
        p.Bk1 ? (const char *)(p.Bk1 + (int64_t)n0 * p.ldb) - 2 * (int64_t)p.kbsplit : nullptr;
    const uint32_t bstep32 = (uint32_t)(32 * p.ldb * 2);
    const int nk = (K + BK - 1) / BK;
    // three K sources (MK): the step's source j, whose K columns start at
    // mk_kb[j]; a step lies in one source (the boundaries are multiples of
    // BK).  Base, row stride and first column are picked with uniform selects;
    // the lane's offset is one 24-bit multiply-add (rows < 256, strides < 2^20).
    struct MkSrc { const bf16_t *base; uint32_t ld; int kb; };
    auto mk_src = [&](int k0, const bf16_t *const *b3, const int64_t *ld3) -> MkSrc {
      const bool s2 = k0 >= p.mk_kb[2], s1 = k0 >= p.mk_kb[1];
      return {s2 ? b3[2] : (s1 ? b3[1] : b3[0]),
              (uint32_t)(s2 ? ld3[2] : (s1 ? ld3[1] : ld3[0])),
              s2 ? p.mk_kb[2] : (s1 ? p.mk_kb[1] : 0)};
    };
    // A tile of K step kt (< nk) into A stage sa (group 0): 8 loads per wave;
    // lanes past M or K read zeros.  No load is issued for steps past the end.
    auto dma_a = [&](int kt, int sa) {
      char *Xs = a_lds + sa * XS;
      const int k0 = kt * BK;
      const int col = k0 + kcol;
      const bool kin = col < K;
      if constexpr (MK) {
        const MkSrc sj = mk_src(k0, p.mk_a, p.mk_lda);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(sj.base + (int64_t)m0 * sj.ld, kMaxRecords);
        const uint32_t base = (uint32_t)(2 * r0) * sj.ld + (uint32_t)(cA * 16) + 2u * (uint32_t)(k0 - sj.kb);
        const uint32_t step = 64u * sj.ld;
  #pragma unroll
        for (int u = 0; u < NI; ++u) {
          const bool ok = kin && 32 * u < arem;
          dma16(rs, Xs + (w4 + 4 * u) * 1024, ok ? base + (uint32_t)u * step : kOOB, 0);
        }
      } else {
        const uint32_t ka = 2u * (uint32_t)k0 + (col >= ksplit ? dA1 : 0u);
  #pragma unroll
        for (int u = 0; u < NI; ++u) {
          const bool ok = kin && 32 * u < arem;
          dma16(rsA, Xs + (w4 + 4 * u) * 1024, ok ? aoff0 + (uint32_t)u * astep + ka : kOOB, 0);
        }
      }
    };
    // B tile of K step kt (< nk) into B stage sb (group 1): 8 loads per wave
    auto dma_b = [&](int kt, int sb) {
      char *Ws = b_lds + sb * WS;
      const int k0 = kt * BK;
      const int col = k0 + kcol;
      const bool kin = col < K;
      if constexpr (MK) {
        const MkSrc sj = mk_src(k0, p.mk_b, p.mk_ldb);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(sj.base + (int64_t)n0 * sj.ld, kMaxRecords);
        const uint32_t base = (uint32_t)(2 * r0) * sj.ld + (uint32_t)(cA * 16) + 2u * (uint32_t)(k0 - sj.kb);
        const uint32_t step = 64u * sj.ld;
  #pragma unroll
        for (int u = 0; u < NI; ++u) {
          const bool ok = kin && 32 * u < brem;
          dma16(rs, Ws + (w4 + 4 * u) * 1024, ok ? base + (uint32_t)u * step : kOOB, 0);
        }
        return;
      }
      // the whole step lies in one K source (kbsplit % BK == 0)
      __amdgpu_buffer_rsrc_t rsK = rsB;
      if (!GU && bk1base != nullptr && k0 >= p.kbsplit) rsK = make_rsrc(bk1base, kMaxRecords);
  #pragma unroll
      for (int u = 0; u < NI; ++u) {
        const int b = w4 + 4 * u;
        if constexpr (GU) {
          const int v = u >> 1;
          const bool ok = kin && 32 * v < brem;
          dma16((u & 1) ? rsB1 : rsB, Ws + b * 1024,
                ok ? boff0 + (uint32_t)v * bstep32 + 2u * (uint32_t)k0 : kOOB, 0);
        } else {
          const bool ok = kin && 32 * u < brem;
          dma16(rsK, Ws + b * 1024, ok ? boff0 + (uint32_t)u * bstep32 + 2u * (uint32_t)k0 : kOOB, 0);
        }
      }
    };

    // ---------------------------------------------------- fragments, MFMAs
    // fragments of K step s (A stage s % 2, B stage s % 3)
    auto rd = [&](int s) {
      const char *Xs = a_lds + (s & 1) * XS, *Ws = b_lds + (s % BSTG) * WS;
  #pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
  #pragma unroll
        for (int i = 0; i < 2; ++i)
          fw[kk][i] = lds_read16(Ws, kc_off<BK>(wn * 64 + i * 32 + l32, 2 * kk + hi32));
  #pragma unroll
        for (int j = 0; j < 4; ++j)
          ft[kk][j] = lds_read16(Xs, kc_off<BK>(wm * 128 + j * 32 + l32, 2 * kk + hi32));
      }
    };

    // ------------------------------------------------------------ K loop
    // Phase t: group t % 2 computes, the other group reads its next fragments.
    // Group 0 reads step s in phase 2s - 1, group 1 in phase 2s.
    //   group 0, memory phase 2s+1: reads step s+1, then loads the A tile of
    //     step s+2 into A stage s % 2 (step s: read in phases 2s-1 and 2s);
    //     drained at the end of its compute phase 2s+2.
    //   group 1, memory phase 2s: drains its B loads of step s+1 (issued two
    //     phases before), loads the B tile of step s+2 into B stage
    //     (s+2) % 3 (step s-1: read in phases 2s-3 and 2s-2), reads step s.
    // Every load therefore targets a stage whose last reads ended before an
    // earlier barrier, and each group's wait drains all of its loads (vmcnt 0)
    // with nothing younger in flight.  (A group-1 wave refilling the stage it
    // had just read, inside the same phase, raced with the other group-1
    // waves still reading it: rare stale fragments, measured.)
    if (grp == 0) {
      dma_a(0, 0);
      if (nk > 1) dma_a(1, 1);
    } else {
      dma_b(0, 0);
      if (nk > 1) dma_b(1, 1);
    }
    wait_vmem();
    pp_barrier();
    if (grp == 0) {
      rd(0);
      lgkm0();
      pp_barrier();
      for (int s = 0; s < nk; ++s) {
        comp();              // step s
        wait_vmem();         // A tile of step s+1 (issued one phase ago)
        pp_barrier();
        // token stage s & 1 was last read in the phase before, so its loads
        // may go first: the store form issues them ahead of the fragment
        // reads (3 % faster there), the SwiGLU forms after them (1 % faster)
        if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_NORM) {
          if (s + 2 < nk) dma_a(s + 2, s & 1);
          if (s + 1 < nk) rd(s + 1);
        } else {
          if (s + 1 < nk) rd(s + 1);
          if (s + 2 < nk) dma_a(s + 2, s & 1);
        }
        lgkm0();
        pp_barrier();
      }
    } else {
      pp_barrier();
      for (int s = 0; s < nk; ++s) {
        wait_vmem();         // B tile of step s+1 (issued two phases ago)
        if (s + 2 < nk) dma_b(s + 2, (s + 2) % BSTG);
        rd(s);
        lgkm0();
        pp_barrier();
        comp();              // step s
        pp_barrier();
      }
    }
  }
  wait_vmem();
  __syncthreads();         // stages free for the epilogue

  // SwiGLU forward with a folded norm: the rows' rstd, requested before the
  // LoRA pass so the epilogue does not wait on them
  float grs[2][4];
  if constexpr (EPI == EPI_SWIGLU_FWD_NORM) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int m = m0 + wm * 128 + h * 64 + it * 16 + (lane >> 2);
        grs[h][it] = m < M ? p.rowscale[m] : 1.f;
      }
  }
  // store with a folded norm: a half's row factors (and raw rows) are all
  // requested before the half is staged
  u32x4 nxv[8];
  float nrs[8], nkk[8];
  auto load_norm = [&](int half) {
    if constexpr (EPI == EPI_STORE_NORM) {
      const int q = lane & 7, n = n0 + wn * 64 + 8 * q;
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int m = m0 + wm * 128 + half * 64 + it * 8 + (lane >> 3);
        const bool ok = m < M && n < N;
        nrs[it] = !ok ? 0.f : p.nrm_x ? p.nrm_rs[m] : p.rowscale ? p.rowscale[m] : 1.f;
        nkk[it] = ok && p.nrm_x ? p.nrm_kk[m] : 0.f;
        nxv[it] = ok && p.nrm_x ? gload16(p.nrm_x + (int64_t)m * N + n) : u32x4{0, 0, 0, 0};
      }
    }
  };
  // SwiGLU backward: a half's saved e, g are all requested before the half
  // is staged
  u32x4 ein[8], gin[8];
  auto load_eg = [&](int half) {
    if constexpr (EPI == EPI_SWIGLU_BWD) {
      const int q = lane & 7, n = n0 + wn * 64 + 8 * q;
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int m = m0 + wm * 128 + half * 64 + it * 8 + (lane >> 3);
        u32x4 e = {0, 0, 0, 0}, g = {0, 0, 0, 0};
        if (m < M && n < N) {
          const int64_t off = (int64_t)m * N + n;
          e = gload16_nt(p.Ein + off);
          g = gload16_nt(p.Gin + off);
        }
        ein[it] = e;
        gin[it] = g;
      }
    }
  };
  // SwiGLU forward with fr_ud: the lane's Ad operand for the H_d partials
  // (row l % 16, the wave's features 8 (l / 16) ..), requested without a
  // branch ahead of the LoRA pass, whose own waits then cover it (a zero
  // operand where it does not apply)
  u32x4 sdh = {0, 0, 0, 0};
  bool sdh_ok = false;
  if constexpr (GU) {
    const int jf = tn * 128 + wn * 32 + 8 * (lane >> 4);
    sdh_ok = p.fr_ud != nullptr && jf < p.gu_f;
    sdh = gload16(sdh_ok ? p.fr_sd + (int64_t)(lane & 15) * p.gu_f + jf : p.epi);
  }
  // ------------------------------------------------ LoRA epilogue pass
  // acc += S . E^T with K = rs: S = s (A_op SIDE^T) [M x rs], E [N x rs]
  // Two 16-column slices per round trip: every load of the pair is issued
  // before its MFMAs (the fragment registers are free by now).
  // With rs_seg (rank blocks of whole 16-column groups) the epilogue operand
  // is block-diagonal.  Fused q/k/v: a tile's columns lie in one projection,
  // whose rows of it are zero outside that projection's block.  Gate/up: the
  // gate rows (i = 0) are zero outside block 0, the up rows outside block 1
  // (with epi_u the two blocks are Bg and Bu as they are).
  const int rs = p.rs;
  int kqb = 0, kqe = rs / 16;
  const int kqs = GU ? p.rs_seg / 16 : 0;   // gate/up: first column group of block 1
  if (!GU && p.rs_seg > 0) {
    const int sgi = (p.nseg2 > 0 && n0 >= p.nseg2) ? 2 : (n0 >= p.nseg1 ? 1 : 0);
    kqb = sgi * (p.rs_seg / 16);
    kqe = kqb + p.rs_seg / 16;
  }
  // gate/up with blocks: does row group i take column group kq
  auto gu_takes = [&](int i, int kq) { return kqs == 0 || (kq < kqs) == (i == 0); };
  for (int kq0 = kqb; kq0 < kqe; kq0 += 2) {
    u32x4 ea[2][2], hb[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kq = kq0 + h;
      const bool qok = kq < kqe;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bf16_t *src;
        bool ok;
        if constexpr (GU) {
          const int j = tn * 128 + wn * 32 + l32;
          ok = j < p.gu_f;
          src = p.epi_u ? (i ? p.epi_u : p.epi) + (int64_t)j * p.rs_seg + (kq - (i ? kqs : 0)) * 16
                        : p.epi + (int64_t)((i ? p.gu_f : 0) + j) * rs + kq * 16;
        } else {
          const int n = n0 + wn * 64 + i * 32 + l32;
          ok = n < N;
          src = p.epi + (int64_t)n * rs + kq * 16;
        }
        u32x4 v = {0, 0, 0, 0};
        if (ok && qok && gu_takes(i, kq)) v = gload16(src + 8 * hi32);
        ea[h][i] = v;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = m0 + wm * 128 + j * 32 + l32;
        u32x4 v = {0, 0, 0, 0};
        if (m < M && qok) v = gload16(p.hglob + (int64_t)m * rs + kq * 16 + 8 * hi32);
        hb[h][j] = v;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (kq0 + h < kqe) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (!gu_takes(i, kq0 + h)) continue;
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(ea[h][i], hb[h][j], acc[i][j]);
        }
      }
    }
  }

  if constexpr (GU) {
    // the Ad operand settled here, where no store is in flight yet (a use in
    // the epilogue would otherwise wait for the epilogue's own stores)
    if (!sdh_ok) sdh = u32x4{0, 0, 0, 0};
    asm volatile("" : "+v"(sdh));
  }

  if constexpr (EPI == EPI_SWIGLU_BWD_RANK) {
    // ---------------------------------- SwiGLU' with the rank-r products
    // Per wave (128 tokens x 64 features), four quarters of 32 tokens: the
    // quarter's dh goes through a private fp32 staging area (8 KB), de, dg
    // and h = silu(e) g are stored and also written as bf16 tiles [32 x 64]
    // (4 KB each, 128-byte rows, chunk ^ (r ^ r / 8) % 8), and 16x16x32
    // MFMAs contract them: over the wave's 64 features with Ad, Bg^T, Bu^T
    // (row reads) and over the quarter's 32 tokens with G_d^T, H_g^T, H_u^T
    // (transpose reads).  Feature sums of the 4 waves that share tokens, and
    // token sums of the 2 waves that share features, are added through LDS
    // in a fixed order and written once per tile.
    constexpr int WREG = 20480;
    char *stg = smem + wave * WREG;
    char *const tl0 = stg + 8192, *const tl1 = stg + 12288, *const tl2 = stg + 16384;
    auto ep_off = [](int r, int c) -> uint32_t { return (uint32_t)(r * 256 + ((c ^ (r & 15)) << 4)); };
    auto tb_off = [](int r, int c) -> uint32_t {
      return (uint32_t)(r * 128 + ((c ^ ((r ^ (r >> 3)) & 7)) << 4));
    };
    const int l16 = lane & 15, g4 = lane >> 4;
    const int fcol0 = n0 + wn * 64, trow0 = m0 + wm * 128;
    const int tiles_n = p.tiles_n;
    f32x4 vd[4], vg[4], vu[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) vd[nb] = vg[nb] = vu[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int q = lane & 7;                       // 8-column group
    const int n = fcol0 + 8 * q;
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      // the quarter's dh (token block jq) into the staging area first: its
      // accumulators are free before the quarter's operands are loaded
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16 &a = acc[i][jq];
          const u32x4 v = {__float_as_uint(a[4 * g]), __float_as_uint(a[4 * g + 1]),
                           __float_as_uint(a[4 * g + 2]), __float_as_uint(a[4 * g + 3])};
          lds_write16(stg, ep_off(l32, 8 * i + 2 * g + hi32), v);
        }
      u32x4 ein[4], gin[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int m = trow0 + jq * 32 + it * 8 + (lane >> 3);
        u32x4 e = {0, 0, 0, 0}, g = {0, 0, 0, 0};
        if (m < M && n < N) {
          const int64_t off = (int64_t)m * N + n;
          e = gload16_nt(p.Ein + off);
          g = gload16_nt(p.Gin + off);
        }
        ein[it] = e;
        gin[it] = g;
      }
      const int tk = trow0 + jq * 32 + 8 * g4;    // token-contraction K block
      u32x4 pd = {0, 0, 0, 0}, pg = pd, pu = pd;
      if (tk < p.fr_ldp) {
        const int64_t o = (int64_t)l16 * p.fr_ldp + tk;
        pd = gload16(p.fr_pd + o);
        pg = gload16(p.fr_pg + o);
        pu = gload16(p.fr_pu + o);
      }
      lgkm0();
      __builtin_amdgcn_wave_barrier();
      // the quarter's loads are settled here, ahead of the row loop: a first
      // use inside the loop's per-lane branches would leave the later rows
      // waiting for the rows' stores as well
      asm volatile("" ::"v"(ein[0]), "v"(ein[1]), "v"(ein[2]), "v"(ein[3]), "v"(gin[0]), "v"(gin[1]),
                   "v"(gin[2]), "v"(gin[3]), "v"(pd), "v"(pg), "v"(pu));
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = it * 8 + (lane >> 3);
        const int m = trow0 + jq * 32 + r;
        const u32x4 a0 = lds_read16(stg, ep_off(r, 2 * q)), a1 = lds_read16(stg, ep_off(r, 2 * q + 1));
        const bool valid = m < M && n < N;
        const float v[8] = {__uint_as_float(a0[0]), __uint_as_float(a0[1]), __uint_as_float(a0[2]),
                            __uint_as_float(a0[3]), __uint_as_float(a1[0]), __uint_as_float(a1[1]),
                            __uint_as_float(a1[2]), __uint_as_float(a1[3])};
        u32x4 dew = {0, 0, 0, 0}, dgw = dew, hw = dew;
        float csum = 0.f;
        if (valid) {
          const u32x4 ev = ein[it], gv = gin[it];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            float de[2], dg[2], hh[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const float e = h2 ? bf16hi(ev[t]) : bf16lo(ev[t]);
              const float gg = h2 ? bf16hi(gv[t]) : bf16lo(gv[t]);
              const float dh = v[2 * t + h2];
              const float sgm = sigmoidf_fast(e);
              dg[h2] = dh * e * sgm;
              de[h2] = dh * gg * sgm * (1.0f + e * (1.0f - sgm));
              hh[h2] = e * sgm * gg;
            }
            dew[t] = pack_bf16x2(de[0], de[1]);
            dgw[t] = pack_bf16x2(dg[0], dg[1]);
            hw[t] = pack_bf16x2(hh[0], hh[1]);
            if (p.cpart)
              csum += bf16lo(dew[t]) * bf16lo(ev[t]) + bf16hi(dew[t]) * bf16hi(ev[t]) +
                      bf16lo(dgw[t]) * bf16lo(gv[t]) + bf16hi(dgw[t]) * bf16hi(gv[t]);
          }
          const int64_t doff = (int64_t)m * p.ldd + n;
          gstore16_nt(p.DE + doff, dew);
          gstore16_nt(p.DG + doff, dgw);
        }
        if (p.cpart) {   // folded RMSNorm: see EPI_SWIGLU_BWD
          csum = sum8_lanes(csum);
          if (q == 0 && m < M) p.cpart[(int64_t)(tn * 4 + wn) * M + m] = csum;
        }
        lds_write16(tl0, tb_off(r, q), hw);
        lds_write16(tl1, tb_off(r, q), dew);
        lds_write16(tl2, tb_off(r, q), dgw);
      }
      lgkm0();
      __builtin_amdgcn_wave_barrier();
      // feature-contraction operands (rows q = l16 of Ad, Bg^T, Bu^T over the
      // wave's features), in flight behind the token contractions
      u32x4 sd[2], sg[2], su[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int nk = fcol0 + 32 * ks + 8 * g4;
        const u32x4 z = {0, 0, 0, 0};
        const bool ok = nk < N;
        const int64_t o = (int64_t)l16 * N + nk;
        sd[ks] = ok ? gload16(p.fr_sd + o) : z;
        sg[ks] = ok ? gload16(p.fr_sg + o) : z;
        su[ks] = ok ? gload16(p.fr_su + o) : z;
      }
      // token contractions: D[q][n] of the wave's four 16-feature blocks
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int col = nb * 16 + 4 * (l16 & 3);
        const int r0 = 8 * g4 + (l16 >> 2);
        const uint32_t o0 = tb_off(r0, col >> 3) + (col & 7) * 2;
        const uint32_t o1 = tb_off(r0 + 4, col >> 3) + (col & 7) * 2;
        const u32x2 h0 = lds_read_tr8(tl0, o0), h1 = lds_read_tr8(tl0, o1);
        const u32x2 d0 = lds_read_tr8(tl1, o0), d1 = lds_read_tr8(tl1, o1);
        const u32x2 x0 = lds_read_tr8(tl2, o0), x1 = lds_read_tr8(tl2, o1);
        vd[nb] = mfma16(pd, u32x4{h0[0], h0[1], h1[0], h1[1]}, vd[nb]);
        vg[nb] = mfma16(pg, u32x4{d0[0], d0[1], d1[0], d1[1]}, vg[nb]);
        vu[nb] = mfma16(pu, u32x4{x0[0], x0[1], x1[0], x1[1]}, vu[nb]);
      }
      // feature contractions: D[q][t] of the quarter's two 16-token blocks
      f32x4 uh[2], ug[2], uu[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        uh[tb] = ug[tb] = uu[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint32_t o = tb_off(tb * 16 + l16, 4 * ks + g4);
          uh[tb] = mfma16(sd[ks], lds_read16(tl0, o), uh[tb]);
          ug[tb] = mfma16(sg[ks], lds_read16(tl1, o), ug[tb]);
          uu[tb] = mfma16(su[ks], lds_read16(tl2, o), uu[tb]);
        }
      }
      // the 4 waves of this token half add their feature sums: product
      // slot (p, tb) of every wave, then wave (wm, wn < 3) sums product wn
      lgkm0();
      auto red_off = [&](int w, int pr, int tb) -> uint32_t {
        return (uint32_t)(w * WREG + ((pr * 2 + tb) * 64 + lane) * 16);
      };
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        *reinterpret_cast<f32x4 *>(smem + red_off(wave, 0, tb)) = uh[tb];
        *reinterpret_cast<f32x4 *>(smem + red_off(wave, 1, tb)) = ug[tb];
        *reinterpret_cast<f32x4 *>(smem + red_off(wave, 2, tb)) = uu[tb];
      }
      __syncthreads();
      if (wn < 3) {
        const int pr = wn;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          f32x4 sum = *reinterpret_cast<const f32x4 *>(smem + red_off(wm, pr, tb));
#pragma unroll
          for (int w2 = 1; w2 < 4; ++w2) {
            const f32x4 o = *reinterpret_cast<const f32x4 *>(smem + red_off(w2 * 2 + wm, pr, tb));
            sum = f32x4{sum[0] + o[0], sum[1] + o[1], sum[2] + o[2], sum[3] + o[3]};
          }
          const int t = trow0 + jq * 32 + tb * 16 + l16;
          if (t < M) {
            float *dst = pr == 0 ? p.fr_ud + ((int64_t)tn * M + t) * 16
                                 : p.fr_ugu + ((int64_t)((pr == 2 ? tiles_n : 0) + tn) * M + t) * 16;
            *reinterpret_cast<f32x4 *>(dst + 4 * g4) = sum;
          }
        }
      }
      __syncthreads();   // staging areas free for the next quarter
    }
    // the 2 waves of this feature block add their token sums: wave wm = 0
    // writes dAd and dBg, wave wm = 1 dBu
    auto vred_off = [&](int w, int pr, int nb) -> uint32_t {
      return (uint32_t)(w * WREG + ((pr * 4 + nb) * 64 + lane) * 16);
    };
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      *reinterpret_cast<f32x4 *>(smem + vred_off(wave, 0, nb)) = vd[nb];
      *reinterpret_cast<f32x4 *>(smem + vred_off(wave, 1, nb)) = vg[nb];
      *reinterpret_cast<f32x4 *>(smem + vred_off(wave, 2, nb)) = vu[nb];
    }
    __syncthreads();
    // Each lane then writes 16 bytes: row q = 4 (l / 16) + e_q of a product,
    // columns nb * 16 + 4 (l % 4) .. +3 for e_q = (l / 4) % 4 -- values of
    // lanes 4 (l % 4) .. +3 of the MFMA layout (lane (n, g) holds q = 4 g ..
    // 4 g + 3 of column n), read back from LDS with one word per lane.
    const int w0 = wn * 2, w1 = wn * 2 + 1;      // the two waves of this feature block
    const int vq = 4 * (lane >> 4) + ((lane >> 2) & 3);   // row q
    const int vc = 4 * (lane & 3);                         // first of 4 columns in the block
#pragma unroll
    for (int pr = 0; pr < 3; ++pr) {
      if ((pr < 2) != (wm == 0)) continue;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int ng = fcol0 + nb * 16 + vc;
        f32x4 v;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          // source lane: column vc + c, group vq / 4, element vq % 4
          const int sl = (vq >> 2) * 16 + vc + c;
          const uint32_t o = (uint32_t)(((pr * 4 + nb) * 64 + sl) * 16 + (vq & 3) * 4);
          v[c] = *reinterpret_cast<const float *>(smem + w0 * WREG + o) +
                 *reinterpret_cast<const float *>(smem + w1 * WREG + o);
        }
        if (ng >= N) continue;   // N % 8 == 0: a 4-column group is all in or all out
        float *dst = pr == 0 ? p.fr_vd + ((int64_t)tm * 16 + vq) * N + ng
                             : p.fr_vgu + ((int64_t)tm * 16 + vq) * 2 * N + (pr == 2 ? N : 0) + ng;
        *reinterpret_cast<f32x4 *>(dst) = v;
      }
    }
  } else {
  // ------------------------------------------------ output
    // A lane holds 4 consecutive output columns of one token row per MFMA
    // block.  Each wave passes its 128 x 64 sub-tile through a private 16 KB
    // LDS region, 64 token rows (fp32) at a time, then reads and writes global
    // memory in 16-byte pieces along rows.  Region row r (0..63) is 256 bytes;
    // 16-byte chunk c (columns 4c .. 4c+3) sits at chunk c ^ (r % 16).
    char *reg = smem + wave * 16384;
    auto ep_off = [](int r, int c) -> uint32_t { return (uint32_t)(r * 256 + ((c ^ (r & 15)) << 4)); };
    // SwiGLU forward with fr_ud: the tile's share of H_d = h Ad^T.  Each wave
    // writes its half's h [64 tokens x 32 features] as a bf16 LDS tile (4 KB
    // past the staging regions, 64-byte rows, chunk c at c ^ (r / 4) % 4) and
    // contracts it over its 32 features with one 16x16x32 MFMA per 16 tokens
    // against Ad; the 4 waves of a token half then add their sums in a fixed
    // order and write them once.
    const bool hd_on = GU && p.fr_ud != nullptr;
    char *const htl = smem + 8 * 16384 + wave * 4096;
    auto ht_off = [](int r, int c) -> uint32_t { return (uint32_t)(r * 64 + ((c ^ ((r >> 2) & 3)) << 4)); };
    const int l16 = lane & 15, g4 = lane >> 4;
    f32x4 uhd[2][4];
  #pragma unroll
    for (int half = 0; half < 2; ++half) {
      load_eg(half);
      load_norm(half);
      // region rows jj * 32 + l32 hold token block j = 2 half + jj
  #pragma unroll
      for (int jj = 0; jj < 2; ++jj)
  #pragma unroll
        for (int i = 0; i < 2; ++i)
  #pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16 &a = acc[i][2 * half + jj];
            const u32x4 v = {__float_as_uint(a[4 * g]), __float_as_uint(a[4 * g + 1]),
                             __float_as_uint(a[4 * g + 2]), __float_as_uint(a[4 * g + 3])};
            lds_write16(reg, ep_off(jj * 32 + l32, 8 * i + 2 * g + hi32), v);
          }
      lgkm0();
      __builtin_amdgcn_wave_barrier();
      // the half's loads are settled here, ahead of the row loop: a first use
      // inside the loop's per-lane branches would leave the later rows
      // waiting for the rows' stores as well
      if constexpr (EPI == EPI_SWIGLU_BWD)
        asm volatile("" ::"v"(ein[0]), "v"(ein[1]), "v"(ein[2]), "v"(ein[3]), "v"(ein[4]), "v"(ein[5]),
                     "v"(ein[6]), "v"(ein[7]), "v"(gin[0]), "v"(gin[1]), "v"(gin[2]), "v"(gin[3]),
                     "v"(gin[4]), "v"(gin[5]), "v"(gin[6]), "v"(gin[7]));
      if constexpr (EPI == EPI_STORE_NORM)
        asm volatile("" ::"v"(nxv[0]), "v"(nxv[1]), "v"(nxv[2]), "v"(nxv[3]), "v"(nxv[4]), "v"(nxv[5]),
                     "v"(nxv[6]), "v"(nxv[7]), "v"(nrs[0]), "v"(nrs[1]), "v"(nrs[2]), "v"(nrs[3]),
                     "v"(nrs[4]), "v"(nrs[5]), "v"(nrs[6]), "v"(nrs[7]), "v"(nkk[0]), "v"(nkk[1]),
                     "v"(nkk[2]), "v"(nkk[3]), "v"(nkk[4]), "v"(nkk[5]), "v"(nkk[6]), "v"(nkk[7]));
      const int mrow0 = m0 + wm * 128 + half * 64;   // token of region row 0
      if constexpr (GU) {
        // region columns 0..31: gate, 32..63: up, features tn*128 + wn*32 + c
        const int f = p.gu_f;
        const int q = lane & 3;                       // 8-feature group
  #pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int r = it * 16 + (lane >> 2);
          const int m = mrow0 + r;
          const int jf = tn * 128 + wn * 32 + 8 * q;
          const u32x4 e0 = lds_read16(reg, ep_off(r, 2 * q)), e1 = lds_read16(reg, ep_off(r, 2 * q + 1));
          const u32x4 g0 = lds_read16(reg, ep_off(r, 8 + 2 * q)), g1 = lds_read16(reg, ep_off(r, 9 + 2 * q));
          u32x4 hw = {0, 0, 0, 0};
          if (m < M && jf < f) {
            float ev[8] = {__uint_as_float(e0[0]), __uint_as_float(e0[1]), __uint_as_float(e0[2]),
                           __uint_as_float(e0[3]), __uint_as_float(e1[0]), __uint_as_float(e1[1]),
                           __uint_as_float(e1[2]), __uint_as_float(e1[3])};
            float gv[8] = {__uint_as_float(g0[0]), __uint_as_float(g0[1]), __uint_as_float(g0[2]),
                           __uint_as_float(g0[3]), __uint_as_float(g1[0]), __uint_as_float(g1[1]),
                           __uint_as_float(g1[2]), __uint_as_float(g1[3])};
            if constexpr (EPI == EPI_SWIGLU_FWD_NORM) {   // folded RMSNorm: the row's rstd
              const float rs = grs[half][it];
  #pragma unroll
              for (int t = 0; t < 8; ++t) {
                ev[t] *= rs;
                gv[t] *= rs;
              }
            }
            u32x4 ew, gw;
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
          if (hd_on) lds_write16(htl, ht_off(r, q), hw);   // zeros outside M x f
        }
        if (hd_on) {
          lgkm0();
          __builtin_amdgcn_wave_barrier();
  #pragma unroll
          for (int tb = 0; tb < 4; ++tb)
            uhd[half][tb] = mfma16(sdh, lds_read16(htl, ht_off(tb * 16 + l16, g4)),
                                   f32x4{0.f, 0.f, 0.f, 0.f});
        }
      } else {
        const int q = lane & 7;                       // 8-column group
        const int n = n0 + wn * 64 + 8 * q;
  #pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int r = it * 8 + (lane >> 3);
          const int m = mrow0 + r;
          const u32x4 a0 = lds_read16(reg, ep_off(r, 2 * q)), a1 = lds_read16(reg, ep_off(r, 2 * q + 1));
          const bool valid = m < M && n < N;
          float v[8] = {__uint_as_float(a0[0]), __uint_as_float(a0[1]), __uint_as_float(a0[2]),
                        __uint_as_float(a0[3]), __uint_as_float(a1[0]), __uint_as_float(a1[1]),
                        __uint_as_float(a1[2]), __uint_as_float(a1[3])};
          if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_NORM) {
            if (!valid) continue;
            if constexpr (EPI == EPI_STORE_NORM) {
              if (!p.nrm_x && p.rowscale) {   // folded RMSNorm: the row's rstd
                const float rs = nrs[it];
  #pragma unroll
                for (int t = 0; t < 8; ++t) v[t] *= rs;
              }
              if (p.nrm_x) {   // RMSNorm input gradient from the folded projections' output
                const u32x4 xv = nxv[it];
                const float rs = nrs[it], kk = nkk[it];
  #pragma unroll
                for (int t = 0; t < 4; ++t) {
                  v[2 * t] = rs * v[2 * t] - kk * bf16lo(xv[t]);
                  v[2 * t + 1] = rs * v[2 * t + 1] - kk * bf16hi(xv[t]);
                }
              }
            }
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
            float csum = 0.f;
            if (valid) {
              const u32x4 ev = ein[it], gv = gin[it];
              u32x4 dew, dgw, hw;
  #pragma unroll
              for (int t = 0; t < 4; ++t) {
                float de[2], dg[2], hh[2];
  #pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                  const float e = h2 ? bf16hi(ev[t]) : bf16lo(ev[t]);
                  const float gg = h2 ? bf16hi(gv[t]) : bf16lo(gv[t]);
                  const float dh = v[2 * t + h2];
                  const float sg = sigmoidf_fast(e);
                  dg[h2] = dh * e * sg;
                  de[h2] = dh * gg * sg * (1.0f + e * (1.0f - sg));
                  hh[h2] = e * sg * gg;
                }
                dew[t] = pack_bf16x2(de[0], de[1]);
                dgw[t] = pack_bf16x2(dg[0], dg[1]);
                hw[t] = pack_bf16x2(hh[0], hh[1]);
                // de e + dg g with de, dg as stored (a folded RMSNorm's row
                // coefficient; unused otherwise)
                if (p.cpart)
                  csum += bf16lo(dew[t]) * bf16lo(ev[t]) + bf16hi(dew[t]) * bf16hi(ev[t]) +
                          bf16lo(dgw[t]) * bf16lo(gv[t]) + bf16hi(dgw[t]) * bf16hi(gv[t]);
              }
              const int64_t doff = (int64_t)m * p.ldd + n;
              gstore16_nt(p.DE + doff, dew);
              gstore16_nt(p.DG + doff, dgw);
              // h = silu(e) g for the rank-r passes that follow (read again
              // right after: a plain store)
              if (p.H) gstore16(p.H + (int64_t)m * N + n, hw);
            }
            if (p.cpart) {
              // the 8 lanes of one row (lanes 8j .. 8j+7) add their sums in a
              // fixed order; every lane takes part (invalid ones add 0)
              csum = sum8_lanes(csum);
              if (q == 0 && m < M) p.cpart[(int64_t)(tn * 4 + wn) * M + m] = csum;
            }
          }
        }
      }
      lgkm0();
      __builtin_amdgcn_wave_barrier();
    }
    if constexpr (GU) {
      if (hd_on) {
        // block b = 4 half + tb of wave w at w * 16 KB + (b * 64 + lane) * 16;
        // wave (wm, wn) sums blocks 2 wn, 2 wn + 1 over the waves wn' * 2 + wm
#pragma unroll
        for (int b = 0; b < 8; ++b)
          *reinterpret_cast<f32x4 *>(smem + wave * 16384 + (b * 64 + lane) * 16) = uhd[b >> 2][b & 3];
        __syncthreads();
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const int b = 2 * wn + bb;
          f32x4 sum = *reinterpret_cast<const f32x4 *>(smem + wm * 16384 + (b * 64 + lane) * 16);
#pragma unroll
          for (int w2 = 1; w2 < 4; ++w2) {
            const f32x4 o =
                *reinterpret_cast<const f32x4 *>(smem + (w2 * 2 + wm) * 16384 + (b * 64 + lane) * 16);
            sum = f32x4{sum[0] + o[0], sum[1] + o[1], sum[2] + o[2], sum[3] + o[3]};
          }
          const int t = m0 + wm * 128 + (b >> 2) * 64 + (b & 3) * 16 + l16;
          if (t < M)
            *reinterpret_cast<f32x4 *>(p.fr_ud + ((int64_t)tn * M + t) * 16 + 4 * g4) = sum;
        }
      }
    }
  }
}

}  // namespace lora
