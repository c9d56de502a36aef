// Device building blocks shared by the liblora kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t bf16_t;  // bf16 storage (bit pattern)

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16x2 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  f32x2_t v = {lo, hi};
  bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

// --------------------------------------------------------------- MFMA -----
__device__ __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ------------------------------------------------------ LDS tile layout ----
// A tile row holds 64 bf16 (128 B) = 8 chunks of 16 B.  The chunk index is
// XOR-swizzled with (row ^ row>>3) & 7 so that both the MFMA fragment reads
// (consecutive rows, same chunk) and the transposing writes of the NN loader
// (rows 8 apart, same chunk) spread over distinct banks.
__device__ __forceinline__ uint32_t swz_off(uint32_t row, uint32_t chunk) {
  return row * 128u + ((chunk ^ ((row ^ (row >> 3)) & 7u)) << 4);
}

__device__ __forceinline__ u32x4 lds_read16(const char *base, uint32_t off) {
  return *reinterpret_cast<const u32x4 *>(base + off);
}
__device__ __forceinline__ void lds_write16(char *base, uint32_t off, const u32x4 &v) {
  *reinterpret_cast<u32x4 *>(base + off) = v;
}

// -------------------------------------------------------- global access ----
__device__ __forceinline__ u32x4 gload16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ u32x2 gload8(const void *p) {
  return *reinterpret_cast<const u32x2 *>(p);
}
__device__ __forceinline__ void gstore8(void *p, const u32x2 &v) {
  *reinterpret_cast<u32x2 *>(p) = v;
}
__device__ __forceinline__ void gstore16(void *p, const u32x4 &v) {
  *reinterpret_cast<u32x4 *>(p) = v;
}
// Streaming (non-temporal) forms for data touched once per pass that would
// only displace reusable lines from L2 and the MALL: the SwiGLU-derivative
// epilogue's e, g reads and de, dg writes.  (The SwiGLU forward's e, g, h
// stores stay cached: h is read again right after.)
__device__ __forceinline__ void gstore16_nt(void *p, const u32x4 &v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ u32x4 gload16_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// ----------------------------------------------------- buffer resources ----
// Raw buffer descriptor (gfx9 layout) over `base`, `bytes` long.  Loads at
// offsets >= bytes return zeros, which the kernels use for every tail: an
// invalid lane gets the offset kOOB.
constexpr uint32_t kOOB = 0x80000000u;
constexpr uint32_t kMaxRecords = 0x7FFFFF00u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
// 16 bytes per lane straight into LDS: lane l writes lds_wave_base + 16 l
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, char *lds_wave_base, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (__attribute__((address_space(3))) void *)lds_wave_base, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0));
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
}
// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, source lane s supplies the 8-byte row at its address; lane i
// receives element i%4 of the rows of lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4.
// With source lane s pointing at W[k0 + s/4][n0 + 4 (s%4) .. +3] of a
// row-major [K x N] tile, lane i gets W[k0 .. k0+3][n0 + i].
__device__ __forceinline__ u32x2 lds_read_tr8(const char *base, uint32_t off) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4 *)((__attribute__((address_space(3))) char *)base + off));
  return __builtin_bit_cast(u32x2, v);
}

// s_waitcnt vmcnt(N) with a compile-time N
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Workgroup barrier without the memory fence of __syncthreads(): the caller
// waits for exactly the loads it needs first (vmcnt / lgkmcnt), so loads of
// later pipeline stages stay in flight across the barrier.  The "memory"
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// 8x8 transpose of bf16: in[i] holds row i (8 values, element j in 16-bit
// lane j), out[j] holds column j (element i = in[i][j]).
__device__ __forceinline__ void transpose8x8(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int dw = j >> 1;
    // selector picks the low (j even) or high (j odd) halves of two words
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // out[j] dword p = (in[2p][j], in[2p+1][j])
      out[j][p] = __builtin_amdgcn_perm(in[2 * p + 1][dw], in[2 * p][dw], sel);
    }
  }
}

// ------------------------------------------------- 4-bit block constants ----
// Where the per-block absmax of a 4-bit weight comes from: plain fp32
// (codes == nullptr) or double-quantised, absmax[b] = table[codes[b]] *
// scale[b / 256] + offset with the product and the sum rounded to fp32
// separately ("Unsloth deep-dive", 1.4: QLoRA also quantises the
// quantisation constants).
struct AbsmaxSrc {
  const float *absmax;      // plain form
  const uint8_t *codes;     // double-quantised form (nullptr: plain)
  const float *table;       // 256 levels
  const float *scale;       // one per 256 blocks
  float offset;
};
__device__ __forceinline__ float absmax_dq(float level, float scale, float offset) {
#pragma clang fp contract(off)
  const float m = level * scale;
  return m + offset;
}
__device__ __forceinline__ float absmax_at(const AbsmaxSrc &s, int64_t b) {
  if (s.codes == nullptr) return s.absmax[b];
  return absmax_dq(s.table[s.codes[b]], s.scale[b >> 8], s.offset);
}

// Sum of x over the 8 lanes 8j .. 8j+7, valid in lane 8j, added as
// ((x0 + x1) + (x2 + x3)) + ((x4 + x5) + (x6 + x7)): DPP lane moves inside
// the VALU, no round trip through the LDS unit.  quad_perm [1,0,3,2] reads
// lane ^ 1, quad_perm [2,3,0,1] lane ^ 2; row_ror:n reads lane (i - n) mod
// 16 of the 16-lane row, so row_ror:12 reads lane (i + 4) mod 16.
__device__ __forceinline__ float sum8_lanes(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x12C, 0xF, 0xF, false));
  return x;
}

// fast logistic with the hardware exp2 / reciprocal
__device__ __forceinline__ float sigmoidf_fast(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

}  // namespace lora
