// Kernels around the main GEMM: rank-r skinny products for the adapter
// gradients, their deterministic reductions, operand preparation, the
// standalone 4-bit decode and the fp32 path.
#pragma once
#include "common.hpp"

namespace lora {

// ---------------------------------------------------------------------------
// skinny NT:  part[ks][t][q] = sum_{k in chunk ks} Z[t][k] * SIDE[q][k]
// Z is bf16 [T x K] (two sources split at K index `ksplit`, for [de | dg]),
// or silu(E) * G recomputed from the saved gate/up activations (ZSWIGLU).
// SIDE is bf16 [RS x K] zero-padded.  Memory-bound: every Z element is read
// once; MFMA 16x16x32 does the rank-RS contraction.
// ---------------------------------------------------------------------------
struct SkinnyNTArgs {
  int T, K, ksplit, kchunk;
  const bf16_t *Z0, *Z1;
  int64_t ldz;
  const bf16_t *E, *G;      // ZSWIGLU sources, ld = ldz
  const bf16_t *side;       // [RS x K], row stride lds (>= K)
  float *part;              // [KS x T x RS]
  int64_t lds;
  // SIDE rows q >= rsplit come from side1 row q - rsplit (same stride): the
  // two adapters of a gate/up pair read in place
  const bf16_t *side1;
  int rsplit;
};

// Block: TB tokens (64 or 128) x one K chunk, stepping 128 columns at a
// time, TB / 16 waves.  Each step's Z tile (TB x 128) and SIDE tile
// (RS x 128) are loaded with row-contiguous 16-byte lanes (a wave
// instruction covers 4 rows x 256 B), kept in registers while the previous
// step's tiles are contracted from LDS, then written to LDS.  Wave w
// contracts tokens 16 w .. 16 w + 15, so the per-wave registers do not
// depend on TB, while the SIDE tile, read once per block and step, costs
// RS / TB of its bytes per Z byte.
// LDS rows are 256 B (16 chunks of 16 B), chunk index XOR (row % 16).
template <int RS, bool ZSWIGLU, int TB = 64>
__global__ __launch_bounds__(TB * 4) void k_skinny_nt(const SkinnyNTArgs a) {
  static_assert(TB == 64 || TB == 128, "64- or 128-token blocks");
  constexpr int NTH = TB * 4;                    // threads
  constexpr int RPI = NTH / 16;                  // rows per load round
  constexpr int NQ = RS / 16;
  constexpr int SL = (RS * 16 + NTH - 1) / NTH;  // side chunks per thread
  __shared__ __attribute__((aligned(16))) char zs[TB * 256];
  __shared__ __attribute__((aligned(16))) char ss[RS * 256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, hi16 = lane >> 4;
  const int t0 = blockIdx.x * TB;
  const int kbeg = blockIdx.y * a.kchunk;
  const int kend = min(a.K, kbeg + a.kchunk);
  const int c = tid & 15, rb = tid >> 4;      // load chunk column, first row
  auto off = [](int row, int chunk) -> uint32_t {
    return (uint32_t)(row * 256 + ((chunk ^ (row & 15)) << 4));
  };
  u32x4 zr[4], sr[SL];
  auto load = [&](int k0) {
    const int k = k0 + 8 * c;
    const bool kin = k < kend;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + rb + RPI * i;
      u32x4 v = {0, 0, 0, 0};
      if (kin && t < a.T) {
        if constexpr (ZSWIGLU) {
          const u32x4 e = gload16(a.E + (int64_t)t * a.ldz + k);
          const u32x4 g = gload16(a.G + (int64_t)t * a.ldz + k);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float e0 = bf16lo(e[w]), e1 = bf16hi(e[w]);
            v[w] = pack_bf16x2(e0 * sigmoidf_fast(e0) * bf16lo(g[w]),
                               e1 * sigmoidf_fast(e1) * bf16hi(g[w]));
          }
        } else {
          // wide ranks stream Z past the caches (a wide pass reads it once,
          // and at the attention workload's [T x f] operands this took the
          // forward's pass over h from 152 to 115 us); narrow ranks keep the
          // cached load, whose operands (X, dY) are read again later
          const bf16_t *src = k < a.ksplit ? a.Z0 + (int64_t)t * a.ldz + k
                                           : a.Z1 + (int64_t)t * a.ldz + (k - a.ksplit);
          if constexpr (RS >= 64) v = gload16_nt(src);
          else v = gload16(src);
        }
      }
      zr[i] = v;
    }
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      const int q = rb + RPI * i;
      u32x4 v = {0, 0, 0, 0};
      if (kin && q < RS)
        v = gload16(q < a.rsplit ? a.side + (int64_t)q * a.lds + k
                                 : a.side1 + (int64_t)(q - a.rsplit) * a.lds + k);
      sr[i] = v;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_write16(zs, off(rb + RPI * i, c), zr[i]);
#pragma unroll
    for (int i = 0; i < SL; ++i)
      if (rb + RPI * i < RS) lds_write16(ss, off(rb + RPI * i, c), sr[i]);
  };
  f32x4 acc[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  load(kbeg);
  store();
  __syncthreads();
  for (int k0 = kbeg; k0 < kend; k0 += 128) {
    const bool more = k0 + 128 < kend;
    if (more) load(k0 + 128);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const u32x4 zf = lds_read16(zs, off(wave * 16 + l16, 4 * kb + hi16));
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb)
        acc[qb] = mfma16(lds_read16(ss, off(qb * 16 + l16, 4 * kb + hi16)), zf, acc[qb]);
    }
    __syncthreads();
    if (more) {
      store();
      __syncthreads();
    }
  }
  // D[q][t]: lane holds q = 16 qb + 4 hi16 .. +3 of token t = t0 + 16 wave + l16
  const int t = t0 + wave * 16 + l16;
  if (t < a.T) {
    float *dst = a.part + ((int64_t)blockIdx.y * a.T + t) * RS;
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb)
      *reinterpret_cast<f32x4 *>(dst + qb * 16 + 4 * hi16) = acc[qb];
  }
}

// For i = t RS + q: out32[t ldo + q] = sum_ks part[ks][i] (fixed order),
// outbf[t ldo + q] = bf16(scale * that sum) (ldo = RS: the [T x RS] layout;
// larger: a column slice of a wider output).  With rowscale, out32 is
// multiplied by rowscale[t] (the bf16 copy is not).
__global__ void k_reduce_side(const float *part, int ks, int64_t count, float scale,
                              float *out32, bf16_t *outbf, const float *rowscale, int RS,
                              int ldo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float s = 0.f;
  for (int k = 0; k < ks; ++k) s += part[(int64_t)k * count + i];
  const int64_t t = i / RS, o = t * ldo + (i - t * RS);
  if (out32) out32[o] = rowscale ? s * rowscale[t] : s;
  if (outbf) {
    const uint32_t w = pack_bf16x2(scale * s, 0.f);
    outbf[o] = (bf16_t)(w & 0xFFFFu);
  }
}

// ---------------------------------------------------------------------------
// skinny TN:  part[ts][q][n] = sum_{t in chunk ts} P[t][q] * Z[t][n]
// P fp32 [T x RS]; Z bf16 [T x N] (two sources split at column `nsplit`,
// for [de | dg]) or silu(E) * G (ZSWIGLU).  The Z tile is transposed 8x8 in
// registers into a t-contiguous LDS layout so the contraction over tokens
// runs on MFMA 16x16x32.
// ---------------------------------------------------------------------------
struct SkinnyTNArgs {
  int T, N, nsplit, tchunk;
  const float *P;           // [T x RS], row stride ldp (>= RS)
  const bf16_t *Z0, *Z1;
  int64_t ldz;
  const bf16_t *E, *G;
  float *part;              // [TS x RS x N]
  int64_t ldp;
};

template <int RS, bool ZSWIGLU>
__global__ __launch_bounds__(256) void k_skinny_tn(const SkinnyTNArgs a) {
  constexpr int NQB = RS / 16;
  // Wide ranks run one wave per SIMD (the accumulators take the register
  // file), so the loop is latency-bound unless the next step's Z rows are in
  // flight during the current step's contractions: those instances keep the
  // raw loads of step t0 + 64 in registers across the step.
  constexpr bool PF = RS >= 64;
  constexpr int NZ = ZSWIGLU ? 2 : 1;        // loaded vectors per row: e, g or z
  __shared__ __attribute__((aligned(16))) char zs[256 * 128];
  __shared__ __attribute__((aligned(16))) char ps[RS * 128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, hi16 = lane >> 4;
  const int n0 = blockIdx.x * 256;
  const int tbeg = blockIdx.y * a.tchunk;
  const int tend = min(a.T, tbeg + a.tchunk);
  f32x4 acc[4][NQB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NQB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int kb = tid >> 5, nb = tid & 31;
  // the raw 16-byte pieces of the thread's 8 rows of step t0 (zero outside)
  auto load_rows = [&](int t0, u32x4 (&raw)[NZ][8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = t0 + kb * 8 + i, n = n0 + nb * 8;
      u32x4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
      if (t < tend && n < a.N) {
        if constexpr (ZSWIGLU) {
          v0 = gload16(a.E + (int64_t)t * a.ldz + n);
          v1 = gload16(a.G + (int64_t)t * a.ldz + n);
        } else {
          const bf16_t *src = n < a.nsplit ? a.Z0 + (int64_t)t * a.ldz + n
                                           : a.Z1 + (int64_t)t * a.ldz + (n - a.nsplit);
          v0 = gload16(src);
        }
      }
      raw[0][i] = v0;
      if constexpr (ZSWIGLU) raw[NZ - 1][i] = v1;
    }
  };
  // P tile [64 tokens x RS] fp32 in units of 4 tokens x 4 ranks: four
  // 16-byte row loads per unit, later transposed into four 8-byte runs of 4
  // tokens
  constexpr int NPU = (RS * 4 + 255) / 256;   // units per thread
  auto load_p = [&](int t0, f32x4 (&pr)[NPU][4]) {
#pragma unroll
    for (int u = 0; u < NPU; ++u) {
      const int idx = tid + 256 * u;
      const int qq = idx >> 4, tq = idx & 15;   // rank quad, token quad
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int t = t0 + 4 * tq + h;
        pr[u][h] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (qq < RS / 4 && t < tend)
          pr[u][h] = *reinterpret_cast<const f32x4 *>(a.P + (int64_t)t * a.ldp + 4 * qq);
      }
    }
  };
  u32x4 raw[NZ][8];
  f32x4 pr[NPU][4];
  if constexpr (PF) {
    if (tbeg < tend) {
      load_rows(tbeg, raw);
      load_p(tbeg, pr);
    }
  }
  for (int t0 = tbeg; t0 < tend; t0 += 64) {
    if constexpr (!PF) {
      load_rows(t0, raw);
      load_p(t0, pr);
    }
    u32x4 rows[8], cols[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (ZSWIGLU) {
        const u32x4 e = raw[0][i], g = raw[NZ - 1][i];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float e0 = bf16lo(e[w]), e1 = bf16hi(e[w]);
          rows[i][w] = pack_bf16x2(e0 * sigmoidf_fast(e0) * bf16lo(g[w]),
                                   e1 * sigmoidf_fast(e1) * bf16hi(g[w]));
        }
      } else {
        rows[i] = raw[0][i];
      }
    }
    transpose8x8(rows, cols);
    u32x2 pv[NPU][4];
#pragma unroll
    for (int u = 0; u < NPU; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pv[u][i] = u32x2{pack_bf16x2(pr[u][0][i], pr[u][1][i]), pack_bf16x2(pr[u][2][i], pr[u][3][i])};
    // the next step's operands, in flight during this step's contractions
    if constexpr (PF) {
      if (t0 + 64 < tend) {
        load_rows(t0 + 64, raw);
        load_p(t0 + 64, pr);
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) lds_write16(zs, swz_off(nb * 8 + j, kb), cols[j]);
#pragma unroll
    for (int u = 0; u < NPU; ++u) {
      const int idx = tid + 256 * u;
      const int qq = idx >> 4, tq = idx & 15;
      if (qq < RS / 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x2 *>(ps + swz_off(4 * qq + i, tq >> 1) + (tq & 1) * 8) = pv[u][i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      u32x4 za[4], pb[NQB];
#pragma unroll
      for (int i = 0; i < 4; ++i) za[i] = lds_read16(zs, swz_off(wave * 64 + i * 16 + l16, 4 * kq + hi16));
#pragma unroll
      for (int j = 0; j < NQB; ++j) pb[j] = lds_read16(ps, swz_off(j * 16 + l16, 4 * kq + hi16));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NQB; ++j) acc[i][j] = mfma16(za[i], pb[j], acc[i][j]);
    }
  }
  // D[n][q]: lane holds 4 consecutive n (rows) of column q
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = n0 + wave * 64 + i * 16 + 4 * hi16;
    if (n >= a.N) continue;
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
      const int q = j * 16 + l16;
      *reinterpret_cast<f32x4 *>(a.part + ((int64_t)blockIdx.y * RS + q) * a.N + n) = acc[i][j];
    }
  }
}

// Sum the TS partials of a TN product, scale, round once to bf16 and scatter
// into the adapter-gradient layout.
//   rowmajor (dA-type): rows q in [0, r) -> out0[q][n], q in [r, 2r) -> out1[q-r][n]
//   transposed (dB-type): out0[n][q] for n < nsplit, q < r;
//                         out1[n-nsplit][q-q1] for n >= nsplit, q1 <= q < q1 + r
// (q1 = r when the second block's rows follow the first's, 0 when both
// blocks start at row 0)
struct ReduceTNArgs {
  const float *part;
  int ts, RS, N, r, nsplit;
  float scale;
  int transposed;
  bf16_t *out0, *out1;
  int q1;
  // optional third block: rowmajor rows q in [2r, 3r); transposed columns
  // n >= nsplit2 with q in [q2, q2 + r)
  bf16_t *out2;
  int nsplit2, q2;
  // optional bf16 column scale (row-major layout: out[q][n] *= colscale[n])
  const bf16_t *colscale;
};
__device__ __forceinline__ void reduce_tn_at(const ReduceTNArgs &a, int64_t i) {
  const int64_t count = (int64_t)a.RS * a.N;
  if (i >= count) return;
  const int q = (int)(i / a.N), n = (int)(i % a.N);
  bf16_t *dst = nullptr;
  if (!a.transposed) {
    if (q < a.r) dst = a.out0 + (int64_t)q * a.N + n;
    else if (q < 2 * a.r && a.out1) dst = a.out1 + (int64_t)(q - a.r) * a.N + n;
    else if (q >= 2 * a.r && q < 3 * a.r && a.out2) dst = a.out2 + (int64_t)(q - 2 * a.r) * a.N + n;
  } else {
    if (n < a.nsplit) {
      if (q < a.r) dst = a.out0 + (int64_t)n * a.r + q;
    } else if (a.out2 && n >= a.nsplit2) {
      if (q >= a.q2 && q < a.q2 + a.r) dst = a.out2 + (int64_t)(n - a.nsplit2) * a.r + (q - a.q2);
    } else if (a.out1 && q >= a.q1 && q < a.q1 + a.r) {
      dst = a.out1 + (int64_t)(n - a.nsplit) * a.r + (q - a.q1);
    }
  }
  if (!dst) return;
  // eight interleaved partial sums (a fixed order) keep eight loads in flight
  float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 8 <= a.ts; k += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = a.part[(int64_t)(k + u) * count + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s8[u] += v[u];
  }
  for (int u = 0; k < a.ts; ++k, ++u) s8[u] += a.part[(int64_t)k * count + i];
  float s = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
  s *= a.scale;
  if (a.colscale && !a.transposed) s *= bf16_to_f32(a.colscale[n]);
  const uint32_t w = pack_bf16x2(s, 0.f);
  *dst = (bf16_t)(w & 0xFFFFu);
}
__global__ void k_reduce_tn(const ReduceTNArgs a) {
  reduce_tn_at(a, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// ---------------------------------------------------------------------------
// dual skinny pass: both rank-r products of one [T x N] operand Z from a
// single read of Z
//   U: part_u[j][t][q]  = sum_{n in column block j} Z[t][n] S[q][n]   (q < RSU)
//   V: part_v[ts][q][n] = sum_{t in token chunk ts} P[q][t] Z[t][n]    (q < RSV)
// Z = [Z0 | Z1]: two column segments (nsplit and N - nsplit columns), each
// with its own S [RSU x segment columns] and P [RSV x ldp] (bf16, zero for
// t >= T); or Z = silu(E) G recomputed from the saved activations (ZSWIGLU,
// one segment).  Column blocks of 256 never straddle the segments; block
// (j, ts) walks its token chunk 64 tokens at a time through LDS: the U part
// reads the tile row-wise (wave w: tokens 16 w .. +15), the V part
// column-wise with transpose reads (wave w: columns 64 w .. +63).
// LDS tile rows are 512 B (32 chunks); chunk index XOR a 4-bit permutation of
// (row % 16) that keeps both the 16-row reads and the 4-row transpose reads
// free of bank conflicts.
// ---------------------------------------------------------------------------
struct DualArgs {
  int T, N, nsplit, tchunk, nb0;   // nb0: column blocks of segment 0
  int64_t ldz;
  const bf16_t *Z0, *Z1, *E, *G;
  const bf16_t *S0, *S1;           // row stride = the segment's column count
  const bf16_t *P0, *P1;
  int ldp;                         // P row stride, a multiple of 64 >= T
  float *part_u;                   // [column blocks x T x RSU]
  float *part_v;                   // [token chunks x RSV x N]
};

// narrow forms are held to 128 VGPRs: 4 workgroups per CU (the LDS limit)
template <int RSU, int RSV, bool ZSWIGLU>
__global__ __launch_bounds__(256, (RSU <= 32 && RSV <= 32) ? 4 : 1) void k_skinny_dual(const DualArgs a) {
  constexpr int NQU = RSU / 16, NQV = RSV / 16;
  constexpr int SL = (RSU * 32 + 255) / 256;   // side chunks per thread
  __shared__ __attribute__((aligned(16))) char zs[64 * 512];
  __shared__ __attribute__((aligned(16))) char ss[RSU * 512];
  // the P tile of the step: [RSV x 64 tokens], 128-byte rows, chunk ^ (q % 8)
  __shared__ __attribute__((aligned(16))) char ps[RSV * 128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int j = blockIdx.x;
  const bool seg1 = j >= a.nb0;
  const int ncol = seg1 ? a.N - a.nsplit : a.nsplit;
  const int c0 = (seg1 ? j - a.nb0 : j) * 256;
  const bf16_t *S = seg1 ? a.S1 : a.S0;
  const bf16_t *P = seg1 ? a.P1 : a.P0;
  const int tbeg = blockIdx.y * a.tchunk, tend = min(a.T, tbeg + a.tchunk);
  auto zoff = [](int r, int c) -> uint32_t {
    const int sw = ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8);
    return (uint32_t)(r * 512 + ((c ^ sw) << 4));
  };
  auto soff = [](int q, int c) -> uint32_t { return (uint32_t)(q * 512 + ((c ^ (q & 15)) << 4)); };
  const int lc = tid & 31, lr = tid >> 5;     // load chunk column, first row

  // side tile of this column block, once
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    const int q = lr + 8 * i;
    if (q < RSU) {
      const int k = c0 + 8 * lc;
      u32x4 v = {0, 0, 0, 0};
      if (k < ncol) v = gload16(S + (int64_t)q * ncol + k);
      lds_write16(ss, soff(q, lc), v);
    }
  }
  // Z tile rows (raw e and g for ZSWIGLU: silu is applied when the tile is
  // written to LDS, so the loads stay in flight behind the step's MFMAs)
  u32x4 zr[8];
  u32x4 gr[ZSWIGLU ? 8 : 1];
  // P tile chunk of this thread: row q = tid / 8, tokens 8 (tid % 8) .. +7
  constexpr int PCH = RSV * 8;   // 16-byte chunks of the P tile
  u32x4 pr = {0, 0, 0, 0};
  auto load = [&](int t0) {
    const int k = c0 + 8 * lc;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = t0 + lr + 8 * i;
      u32x4 v = {0, 0, 0, 0}, w = {0, 0, 0, 0};
      if (t < tend && k < ncol) {
        if constexpr (ZSWIGLU) {
          v = gload16(a.E + (int64_t)t * a.ldz + k);
          w = gload16(a.G + (int64_t)t * a.ldz + k);
        } else {
          v = gload16((seg1 ? a.Z1 : a.Z0) + (int64_t)t * a.ldz + k);
        }
      }
      zr[i] = v;
      if constexpr (ZSWIGLU) gr[i] = w;
    }
    // P rows are zero past T up to ldp (a multiple of 64), so the whole
    // 64-token tile is in bounds
    if (tid < PCH) pr = gload16(P + (int64_t)(tid >> 3) * a.ldp + t0 + 8 * (tid & 7));
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4 v = zr[i];
      if constexpr (ZSWIGLU) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float e0 = bf16lo(zr[i][w]), e1 = bf16hi(zr[i][w]);
          v[w] = pack_bf16x2(e0 * sigmoidf_fast(e0) * bf16lo(gr[i][w]),
                             e1 * sigmoidf_fast(e1) * bf16hi(gr[i][w]));
        }
      }
      lds_write16(zs, zoff(lr + 8 * i, lc), v);
    }
    if (tid < PCH) {
      const int q = tid >> 3, c = tid & 7;
      lds_write16(ps, (uint32_t)(q * 128 + ((c ^ (q & 7)) << 4)), pr);
    }
  };

  f32x4 vacc[4][NQV];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int qb = 0; qb < NQV; ++qb) vacc[nb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  load(tbeg);
  store();
  __syncthreads();
  for (int t0 = tbeg; t0 < tend; t0 += 64) {
    const bool more = t0 + 64 < tend;
    if (more) load(t0 + 64);
    // U: tokens t0 + 16 wave + l16, all 256 columns of the block
    f32x4 uacc[NQU];
#pragma unroll
    for (int qb = 0; qb < NQU; ++qb) uacc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const u32x4 zf = lds_read16(zs, zoff(wave * 16 + l16, 4 * kb + g4));
#pragma unroll
      for (int qb = 0; qb < NQU; ++qb)
        uacc[qb] = mfma16(lds_read16(ss, soff(qb * 16 + l16, 4 * kb + g4)), zf, uacc[qb]);
    }
    // V: columns 64 wave .. +63, the 64 tokens of the tile
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 pf[NQV];
#pragma unroll
      for (int qb = 0; qb < NQV; ++qb) {
        const int q = qb * 16 + l16, c = 4 * kb + g4;
        pf[qb] = lds_read16(ps, (uint32_t)(q * 128 + ((c ^ (q & 7)) << 4)));
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        // lane l16 of group g4: column 64 wave + 16 nb + l16, tokens
        // 32 kb + 8 g4 .. +7 (two 4-token transpose reads)
        const int n = wave * 64 + nb * 16 + 4 * (l16 & 3);
        const int r0 = 32 * kb + 8 * g4 + (l16 >> 2);
        const u32x2 lo = lds_read_tr8(zs, zoff(r0, n >> 3) + (n & 7) * 2);
        const u32x2 hi = lds_read_tr8(zs, zoff(r0 + 4, n >> 3) + (n & 7) * 2);
        const u32x4 za = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int qb = 0; qb < NQV; ++qb) vacc[nb][qb] = mfma16(za, pf[qb], vacc[nb][qb]);
      }
    }
    // U partial: lane holds q = 16 qb + 4 g4 .. +3 of token t
    const int t = t0 + wave * 16 + l16;
    if (t < tend) {
      float *dst = a.part_u + ((int64_t)j * a.T + t) * RSU;
#pragma unroll
      for (int qb = 0; qb < NQU; ++qb)
        *reinterpret_cast<f32x4 *>(dst + qb * 16 + 4 * g4) = uacc[qb];
    }
    __syncthreads();
    if (more) {
      store();
      __syncthreads();
    }
  }
  // V partial: lane holds columns 16 nb + 4 g4 .. +3 (of the wave's 64) of row q
  const int colbase = seg1 ? a.nsplit : 0;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int n = c0 + wave * 64 + nb * 16 + 4 * g4;
    if (n >= ncol) continue;
#pragma unroll
    for (int qb = 0; qb < NQV; ++qb) {
      const int q = qb * 16 + l16;
      *reinterpret_cast<f32x4 *>(a.part_v + ((int64_t)blockIdx.y * RSV + q) * a.N + colbase + n) =
          vacc[nb][qb];
    }
  }
}

// out32[t][qo], outbf[t][qo] = bf16(scale * out32), qo < RSout: with two
// segments, qo < r sums segment 0's column blocks at q = qo, r <= qo < 2r
// sums segment 1's at q = qo - r; with one, qo < RSU sums all blocks.
// Everything else is 0.  Fixed summation order.
struct ReduceUArgs {
  const float *part;
  int T, RSU, RSout, r, nseg, nb0, nb1;
  float scale;
  float *out32;
  bf16_t *outbf;
  const float *rowscale;   // optional: out32[t][.] *= rowscale[t] (not outbf)
};
__device__ __forceinline__ void reduce_dual_u_at(const ReduceUArgs &a, int64_t i) {
  if (i >= (int64_t)a.T * a.RSout) return;
  const int t = (int)(i / a.RSout), qo = (int)(i % a.RSout);
  int q = qo, jb = 0, je = a.nb0;
  bool ok = qo < a.RSU;
  if (a.nseg == 2) {
    const bool s1 = qo >= a.r;
    q = s1 ? qo - a.r : qo;
    jb = s1 ? a.nb0 : 0;
    je = s1 ? a.nb0 + a.nb1 : a.nb0;
    ok = qo < 2 * a.r;
  }
  // eight interleaved partial sums (a fixed order): a thread has eight loads
  // in flight, which the long sums (one partial per 128- or 256-column tile)
  // need to approach the HBM rate
  float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (ok) {
    const float *src = a.part + (int64_t)t * a.RSU + q;
    const int64_t stride = (int64_t)a.T * a.RSU;
    int jj = jb;
    for (; jj + 8 <= je; jj += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = src[(int64_t)(jj + u) * stride];
#pragma unroll
      for (int u = 0; u < 8; ++u) s8[u] += v[u];
    }
    for (int u = 0; jj < je; ++jj, ++u) s8[u] += src[(int64_t)jj * stride];
  }
  const float s = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
  if (a.out32) a.out32[i] = a.rowscale ? s * a.rowscale[t] : s;
  if (a.outbf) {
    const uint32_t w = pack_bf16x2(a.scale * s, 0.f);
    a.outbf[i] = (bf16_t)(w & 0xFFFFu);
  }
}
__global__ void k_reduce_dual_u(const ReduceUArgs a) {
  reduce_dual_u_at(a, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// Independent reductions in one launch (each a launch of its own costs more
// than its few microseconds of work): the U-type jobs first, then the TN-type
// jobs, job j on blocks [start[j], start[j + 1]).
struct ReduceBatch {
  ReduceUArgs u[2];
  ReduceTNArgs v[2];
  int nu, nv;
  int64_t start[5];
};
__global__ void k_reduce_batch(const ReduceBatch b) {
  int j = 0;
  while (j + 1 < b.nu + b.nv && (int64_t)blockIdx.x >= b.start[j + 1]) ++j;
  const int64_t i = ((int64_t)blockIdx.x - b.start[j]) * blockDim.x + threadIdx.x;
  if (j < b.nu) reduce_dual_u_at(b.u[j], i);
  else reduce_tn_at(b.v[j - b.nu], i);
}

// out[q][t] = bf16(in[t][qoff + q]) for q < nq, t < T; 0 elsewhere in
// [RSout x ldp]; up to three such copies (same T, RSout, ldp) in one launch,
// copy c on elements [c RSout ldp, (c + 1) RSout ldp)
struct PackJob {
  const float *in;
  int ldin, qoff, nq;
  bf16_t *out;
};
struct PackBatch {
  PackJob j[3];
  int n, T, RSout, ldp;
};
__global__ void k_pack_pt(const PackBatch b) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)b.RSout * b.ldp;
  if (i >= b.n * per) return;
  const PackJob &jb = b.j[i / per];
  const int64_t e = i % per;
  const int q = (int)(e / b.ldp), t = (int)(e % b.ldp);
  float v = 0.f;
  if (q < jb.nq && t < b.T) v = jb.in[(int64_t)t * jb.ldin + jb.qoff + q];
  const uint32_t w = pack_bf16x2(v, 0.f);
  jb.out[e] = (bf16_t)(w & 0xFFFFu);
}

// ---------------------------------------------------------------------------
// operand preparation (tiny, bf16 copies with zero padding)
// Up to three sources, stacked: source i fills rows (side) or columns (epi)
// q in [i r, (i+1) r).
// side[q][k], q < RS, k < K:
//   !tr: q in block i -> src_i[q - i r][k] (ld K)
//    tr: k in [split_i, split_{i+1}) (split_0 = 0, split_3 = K) and q in block
//        i -> src_i[k - split_i][q - i r] (ld r)
// epi[row][q], row < rows, q < RS:
//   !tr (from B [rows x r]): row in [split_i, split_{i+1}) and q in block i ->
//        src_i[row - split_i][q - i r]
//    tr (from A [r x rows]): q in block i -> src_i[q - i r][row]
// Every other element is zero.  With two sources split_2 = K (or rows).
// ---------------------------------------------------------------------------
// All the small operand copies of one call in a single launch: block b
// works on the job whose block range [start[j], start[j+1]) holds b.
struct PrepJob {
  bf16_t *dst;
  const bf16_t *src0, *src1, *src2;
  int kind;            // 0: side [a = RS x b = K], 1: epi [a = rows x b = RS]
  int a, b, r, split, split2, tr;
  // optional bf16 scale per in_feature of an adapter A (side !tr: per k;
  // epi tr: per row), applied as one fp32 multiply rounded to bf16: the
  // operand becomes A diag(colscale)
  const bf16_t *colscale;
};
constexpr int kMaxPrepJobs = 8;
struct PrepBatch {
  PrepJob job[kMaxPrepJobs];
  unsigned start[kMaxPrepJobs + 1];
  int njobs;
};
__device__ __forceinline__ bf16_t prep_at(const PrepJob &jb, int64_t i) {
  const int r = jb.r;
  const bf16_t *src[3] = {jb.src0, jb.src1, jb.src2};
  bf16_t v = 0;
  if (jb.kind == 0) {   // side[q][k]
    const int K = jb.b, q = (int)(i / K), k = (int)(i % K);
    const int blk = q / r;
    if (blk < 3 && src[blk]) {
      if (!jb.tr) {
        v = src[blk][(int64_t)(q - blk * r) * K + k];
        if (jb.colscale)
          v = (bf16_t)(pack_bf16x2(bf16_to_f32(v) * bf16_to_f32(jb.colscale[k]), 0.f) & 0xFFFFu);
      } else {
        const int lo = blk == 0 ? 0 : (blk == 1 ? jb.split : jb.split2);
        const int hi = blk == 0 ? jb.split : (blk == 1 ? (jb.src2 ? jb.split2 : K) : K);
        if (k >= lo && k < hi) v = src[blk][(int64_t)(k - lo) * r + (q - blk * r)];
      }
    }
  } else {              // epi[row][q]
    const int rows = jb.a, RS = jb.b, row = (int)(i / RS), q = (int)(i % RS);
    const int blk = q / r;
    if (blk < 3 && src[blk]) {
      if (!jb.tr) {
        const int lo = blk == 0 ? 0 : (blk == 1 ? jb.split : jb.split2);
        const int hi = blk == 0 ? jb.split : (blk == 1 ? (jb.src2 ? jb.split2 : rows) : rows);
        if (row >= lo && row < hi) v = src[blk][(int64_t)(row - lo) * r + (q - blk * r)];
      } else {
        v = src[blk][(int64_t)(q - blk * r) * rows + row];
        if (jb.colscale)
          v = (bf16_t)(pack_bf16x2(bf16_to_f32(v) * bf16_to_f32(jb.colscale[row]), 0.f) & 0xFFFFu);
      }
    }
  }
  return v;
}
// A thread writes 8 consecutive elements of a row (one 16-byte store) when
// the row length b is a multiple of 8, else one element.
__global__ __launch_bounds__(256) void k_prep(const PrepBatch pb) {
  int j = 0;
  while (j + 1 < pb.njobs && blockIdx.x >= pb.start[j + 1]) ++j;
  const PrepJob &jb = pb.job[j];
  const int64_t u = (int64_t)(blockIdx.x - pb.start[j]) * 256 + threadIdx.x;
  const int64_t cnt = (int64_t)jb.a * jb.b;
  if (jb.b % 8 == 0) {
    const int64_t i = u * 8;
    if (i >= cnt) return;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)prep_at(jb, i + 2 * e) | ((uint32_t)prep_at(jb, i + 2 * e + 1) << 16);
    gstore16(jb.dst + i, u32x4{w[0], w[1], w[2], w[3]});
  } else {
    if (u >= cnt) return;
    jb.dst[u] = prep_at(jb, u);
  }
}

// ---------------------------------------------------------------------------
// standalone 4-bit decode.  A wave decodes 2048 consecutive elements in
// four passes; in each pass lane l takes code bytes 4 l .. 4 l + 3 of the
// pass's 256 (8 elements, one 64-element block constant) and stores their
// 16 bytes of bf16, so every load instruction covers 256 contiguous bytes
// and every store 1 KB.  total is a multiple of 64.  HBM-bound.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_dequant4(const uint8_t *codes, const AbsmaxSrc absmax,
                                                  const float *codebook, int64_t total,
                                                  bf16_t *out) {
  __shared__ float2 cbt[256];
  cbt[threadIdx.x] = make_float2(codebook[threadIdx.x & 15], codebook[threadIdx.x >> 4]);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t e0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2048 + lane * 8;
  uint32_t c[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int64_t e = e0 + w * 512;
    c[w] = e < total ? *reinterpret_cast<const uint32_t *>(codes + e / 2) : 0u;
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int64_t e = e0 + w * 512;
    if (e >= total) break;
    const float am = absmax_at(absmax, e >> 6);
    u32x4 o;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float2 cv = cbt[(c[w] >> (8 * b)) & 0xFFu];
      o[b] = pack_bf16x2(cv.x * am, cv.y * am);
    }
    gstore16(out + e, o);
  }
}

// ---------------------------------------------------------------------------
// Transposed copies of a frozen base weight for the backward dX GEMMs, so
// they read the weight K-contiguous like the forward GEMMs.  HBM-bound.
//   k_transpose_bf16: out[c * ld_out + r] = in[r * ld_in + c]
//   k_dequant4_t:     out[c * ld_out + r] = decode(W)[r][c]  (4-bit W [rows x cols])
// rows and cols are multiples of 8 (cols of 64 for the 4-bit form).  A thread
// moves 8 rows x 8 columns (transpose) or 8 rows x 32 columns (decode)
// through registers with 8 x 8 register transposes; a wave's loads and
// stores cover 128-byte row segments.  Block b covers column block b % ncb
// and row block b / ncb (a 1-D grid, so neither extent is capped at 65535).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_transpose_bf16(const bf16_t *in, int rows, int cols,
                                                        int64_t ld_in, bf16_t *out,
                                                        int64_t ld_out, int ncb) {
  const int cc = threadIdx.x & 7, rb = threadIdx.x >> 3;
  const int c0 = (int)(blockIdx.x % (unsigned)ncb) * 64 + cc * 8;
  const int r0 = (int)(blockIdx.x / (unsigned)ncb) * 256 + rb * 8;
  if (c0 >= cols || r0 >= rows) return;
  u32x4 v[8], t[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = gload16(in + (int64_t)(r0 + i) * ld_in + c0);
  transpose8x8(v, t);
#pragma unroll
  for (int j = 0; j < 8; ++j) gstore16(out + (int64_t)(c0 + j) * ld_out + r0, t[j]);
}

__global__ __launch_bounds__(256) void k_dequant4_t(const uint8_t *codes, const AbsmaxSrc absmax,
                                                    const float *codebook, int rows, int cols,
                                                    bf16_t *out, int64_t ld_out, int ncb) {
  __shared__ float2 cbt[256];
  cbt[threadIdx.x] = make_float2(codebook[threadIdx.x & 15], codebook[threadIdx.x >> 4]);
  __syncthreads();
  const int cc = threadIdx.x & 7, rb = threadIdx.x >> 3;
  const int c0 = (int)(blockIdx.x % (unsigned)ncb) * 256 + cc * 32;   // 16 code bytes
  const int r0 = (int)(blockIdx.x / (unsigned)ncb) * 256 + rb * 8;
  if (c0 >= cols || r0 >= rows) return;
  u32x4 v[4][8];   // [8-column group][row]
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t e0 = (int64_t)(r0 + i) * cols + c0;   // flat element index
    const u32x4 c = gload16(codes + e0 / 2);
    const float am = absmax_at(absmax, e0 >> 6);
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float2 cv = cbt[(c[w] >> (8 * b)) & 0xFFu];
        v[w][i][b] = pack_bf16x2(cv.x * am, cv.y * am);
      }
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    u32x4 t[8];
    transpose8x8(v[w], t);
#pragma unroll
    for (int j = 0; j < 8; ++j) gstore16(out + (int64_t)(c0 + 8 * w + j) * ld_out + r0, t[j]);
  }
}

// [T x (n0 + n1 + n2)] <- [src0 | src1 | src2] row by row (bf16, column
// counts multiples of 8; 16 bytes per thread)
__global__ __launch_bounds__(256) void k_concat3(const bf16_t *src0, const bf16_t *src1,
                                                 const bf16_t *src2, int n0, int n1, int n2,
                                                 int64_t T, bf16_t *dst) {
  const int N8 = (n0 + n1 + n2) / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * N8) return;
  const int64_t t = i / N8;
  const int c = (int)(i % N8) * 8;
  const bf16_t *src;
  if (c < n0) src = src0 + t * n0 + c;
  else if (c < n0 + n1) src = src1 + t * n1 + (c - n0);
  else src = src2 + t * n2 + (c - n0 - n1);
  gstore16(dst + t * (n0 + n1 + n2) + c, gload16(src));
}

// ---------------------------------------------------------------------------
// Merged weight W' = W + ss * B A (ss = sign * alpha / r): one 64 x 64
// output tile per workgroup; the tile's B rows and A columns are staged in
// LDS as fp32, each thread forms 2 rows x 8 columns of B A (fp32 FMA, fixed
// order over r) and adds them to W (dense bf16 / fp32, or 4-bit decoded to
// bf16 first), rounding once to the output dtype.  HBM-bound.
// ---------------------------------------------------------------------------
struct MergeArgs {
  int n, k, r, ncb;            // ncb: 64-column blocks
  float ss;                    // sign * alpha / r
  int f32;                     // 1: W, A, B, out are fp32; 0: bf16
  const void *W;               // dense weight (NULL for 4-bit)
  const uint8_t *codes;        // 4-bit weight
  AbsmaxSrc absmax;
  const float *codebook;
  const void *A, *B;
  void *out;
};
__global__ __launch_bounds__(256) void k_lora_merge(const MergeArgs a) {
  __shared__ float bs[64][129];
  __shared__ float as_[128][64];
  const int tid = threadIdx.x;
  const int i0 = (int)(blockIdx.x / (unsigned)a.ncb) * 64;
  const int j0 = (int)(blockIdx.x % (unsigned)a.ncb) * 64;
  auto ld = [&](const void *base, int64_t idx) -> float {
    return a.f32 ? reinterpret_cast<const float *>(base)[idx]
                 : __uint_as_float((uint32_t)reinterpret_cast<const bf16_t *>(base)[idx] << 16);
  };
  for (int e = tid; e < 64 * a.r; e += 256) {
    const int ii = e / a.r, q = e % a.r, i = i0 + ii;
    bs[ii][q] = i < a.n ? ld(a.B, (int64_t)i * a.r + q) : 0.f;
  }
  for (int e = tid; e < a.r * 64; e += 256) {
    const int q = e >> 6, jj = e & 63, j = j0 + jj;
    as_[q][jj] = j < a.k ? ld(a.A, (int64_t)q * a.k + j) : 0.f;
  }
  __syncthreads();
  const int jj0 = (tid & 7) * 8, ii0 = (tid >> 3) * 2;
  for (int rr = 0; rr < 2; ++rr) {
    const int ii = ii0 + rr, i = i0 + ii;
    if (i >= a.n) continue;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < a.r; ++q) {
      const float b = bs[ii][q];
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = fmaf(b, as_[q][jj0 + c], acc[c]);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int j = j0 + jj0 + c;
      if (j >= a.k) break;
      const int64_t idx = (int64_t)i * a.k + j;
      float w;
      if (a.codes) {   // 4-bit: decode to bf16 (fp32 product, rounded once)
        const uint32_t byte = a.codes[idx >> 1];
        const uint32_t code = (idx & 1) ? (byte >> 4) : (byte & 15u);
        const uint32_t wb = pack_bf16x2(a.codebook[code] * absmax_at(a.absmax, idx >> 6), 0.f);
        w = bf16lo(wb);
      } else {
        w = ld(a.W, idx);
      }
      const float v = w + a.ss * acc[c];
      if (a.f32) {
        reinterpret_cast<float *>(a.out)[idx] = v;
      } else {
        reinterpret_cast<bf16_t *>(a.out)[idx] = (bf16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 path: generic strided GEMM with fp32 FMA (no matrix cores, so the
// arithmetic stays IEEE fp32):
//   C[m][n] = alpha * sum_k A(m,k) B(k,n) + beta * C[m][n]
//   A(m,k) = A[m*sam + k*sak], B(k,n) = B[k*sbk + n*sbn], C ld = ldc
// 64 x 64 tiles, 256 threads with 4 x 4 outputs each, K step 16 via LDS.
// ---------------------------------------------------------------------------
struct F32GemmArgs {
  int M, N, K;
  const float *A;
  int64_t sam, sak;
  const float *B;
  int64_t sbk, sbn;
  float *C;
  int64_t ldc;
  float alpha, beta;
};
__global__ __launch_bounds__(256) void k_gemm_f32(const F32GemmArgs a) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 1];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tr = tid / 16, tc = tid % 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < a.K; k0 += 16) {
    for (int e = tid; e < 16 * 64; e += 256) {
      const int kk = e / 64, mm = e % 64;
      const int m = m0 + mm, k = k0 + kk;
      As[kk][mm] = (m < a.M && k < a.K) ? a.A[(int64_t)m * a.sam + (int64_t)k * a.sak] : 0.f;
      const int n = n0 + mm;
      Bs[kk][mm] = (n < a.N && k < a.K) ? a.B[(int64_t)k * a.sbk + (int64_t)n * a.sbn] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][tr * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tc * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + tr * 4 + i;
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tc * 4 + j;
      if (n >= a.N) continue;
      float *c = a.C + (int64_t)m * a.ldc + n;
      const float v = a.alpha * acc[i][j];
      *c = (a.beta == 0.f) ? v : v + a.beta * *c;
    }
  }
}

// h = silu(e) * g (fp32, accurate exp)
__global__ void k_swiglu_f32(const float *e, const float *g, float *h, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const float z = e[i];
  h[i] = z / (1.0f + expf(-z)) * g[i];
}
// de = dh g sig (1 + e (1 - sig)), dg = dh e sig (fp32)
__global__ void k_swiglu_bwd_f32(const float *e, const float *g, const float *dh, float *de,
                                 float *dg, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const float z = e[i], sg = 1.0f / (1.0f + expf(-z));
  de[i] = dh[i] * g[i] * sg * (1.0f + z * (1.0f - sg));
  dg[i] = dh[i] * z * sg;
}

// ---------------------------------------------------------------------------
// RMSNorm folded into the projections that follow it
// ---------------------------------------------------------------------------
// out[i][j] = bf16(W[i][j] * w[j]): the frozen norm weight folded into a
// frozen base weight [n x k] (one fp32 multiply, rounded once).  8 elements
// per thread.
__global__ __launch_bounds__(256) void k_fold_colscale(const bf16_t *W, const bf16_t *w, int64_t n,
                                                       int64_t k, bf16_t *out) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // 8-element group
  if (g * 8 >= n * k) return;
  const int64_t j0 = (g * 8) % k;   // k % 8 == 0: a group stays inside one row
  const u32x4 a = gload16(W + g * 8), b = gload16(w + j0);
  u32x4 o;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    o[t] = pack_bf16x2(bf16lo(a[t]) * bf16lo(b[t]), bf16hi(a[t]) * bf16hi(b[t]));
  gstore16(out + g * 8, o);
}

// Coefficient of x in the RMSNorm input gradient, from the down-projection
// backward's per-row partial sums S_p[t] of de e + dg g over column blocks:
//   kk[t] = rstd[t]^2 (sum_p S_p[t]) / d     (fixed summation order)
// (sum_j gn_j x_j = S / rstd with gn = dXn w the gradient the folded
// projections return, so rstd^3 x (gn . x) / d = kk x.)
// Block: 64 rows, 16 waves; wave w adds the partials p = w (mod 16) of its
// lane's row, the 16 wave sums are then added in wave order.
__global__ __launch_bounds__(1024) void k_norm_coef(const float *part, int np, int T,
                                                    const float *rstd, float inv_d, float *kk) {
  __shared__ float red[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = blockIdx.x * 64 + lane;
  float s = 0.f;
  if (t < T)
    for (int p = w; p < np; p += 16) s += part[(int64_t)p * T + t];
  red[w][lane] = s;
  __syncthreads();
  if (w == 0 && t < T) {
    float S = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) S += red[i][lane];
    const float r = rstd[t];
    kk[t] = r * r * S * inv_d;
  }
}

}  // namespace lora
