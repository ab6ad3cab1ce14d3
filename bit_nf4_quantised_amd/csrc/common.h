// Device helpers shared by the NF4 kernels (gfx950 / CDNA4, wave64).
//
// Storage format ("QLoRA, explained", Blockwise absmax quantisation; NormalFloat 4; Double
// quantisation; Minimal implementation):
//   * W is N x K row-major and is cut into blocks of 64 consecutive values (K % 64 == 0, so a block
//     never straddles a row);
//   * packed[j] holds the 4-bit code indices of elements 2j (high nibble) and 2j+1 (low nibble);
//   * scale_q[b] is the OCP E4M3 code of c1[b] / c2[g], g = b / 256; scale_c2[g] is fp32.
// Dequantisation order: c1' = fl32(e4m3(scale_q) * c2), w~ = bf16_rne(fl32(q[idx] * c1')).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4 {

constexpr int kBlock = 64;     // values per absmax block
constexpr int kGroup = 256;    // blocks per second-level constant

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

// The 16 NF4 codes, ascending, as float32 bit patterns: standard-normal quantiles with the
// tail probability 929/960, halves built separately around an exact zero (index 7), divided by
// the top quantile so the ends are exactly -1 and +1.
#define NF4_CODE_BITS                                                                     \
  0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu, 0xbe91a24bu, 0xbe3d353du, 0xbdba7869u, \
      0x00000000u, 0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u, 0x3ee1a4b5u,           \
      0x3f1007a9u, 0x3f3913b0u, 0x3f800000u

__device__ __forceinline__ float code_value(int i) {
  constexpr uint32_t bits[16] = {NF4_CODE_BITS};
  return __uint_as_float(bits[i]);
}

// OCP E4M3 decode of a code in [0x00, 0x7E] (sign bit clear): exponent field 0 is subnormal
// m * 2^-9, otherwise (8 + m) * 2^(e - 10). Built from bits, so it is exact.
__device__ __forceinline__ float e4m3_decode(uint32_t code) {
  uint32_t e = (code >> 3) & 15u, m = code & 7u;
  float normal = __uint_as_float(((e + 120u) << 23) | (m << 20));
  float sub = (float)m * 0x1p-9f;
  return e ? normal : sub;
}

// Round-to-nearest-even pack of two floats into a bf16 pair (lo in bits 0..15).
// gfx950 has v_cvt_pk_bf16_f32, which rounds to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// ------------------------------------------------------------------------------------------
// Per-block bf16 lookup table and byte-permute dequantisation.
//
// For one block the 16 possible dequantised values T[i] = bf16(fl32(q[i] * c1')) are computed
// once and split into byte planes: lo[0..3] hold the low bytes of T[0..15], hi[0..3] the high
// bytes. v_perm_b32 picks a byte out of 8 by a selector 0..7 and yields 0xFF for selectors >= 13;
// two perms ANDed therefore look up a 16-entry table: selector sA = idx (idx < 8) or >= 0x48
// (idx >= 8), sB = sA ^ 0x48 = idx - 8 (idx >= 8) or >= 0x48 (idx < 8).
struct BlockLut {
  uint32_t lo[4], hi[4];
};

// The 16 values a 4-bit index selects (NF4, FP4 or INT4, ascending; a 15-value codebook repeats
// its last value at index 15), passed to kernels by value in their arguments.
struct Codes {
  float v[16];
};

__device__ __forceinline__ BlockLut make_lut(float c1p, const float (&q)[16]) {
  uint32_t p[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) p[k] = pack_bf16x2(__fmul_rn(q[2 * k], c1p), __fmul_rn(q[2 * k + 1], c1p));
  BlockLut t;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    t.lo[k] = __builtin_amdgcn_perm(p[2 * k + 1], p[2 * k], 0x06040200u);
    t.hi[k] = __builtin_amdgcn_perm(p[2 * k + 1], p[2 * k], 0x07050301u);
  }
  return t;
}

__device__ __forceinline__ BlockLut make_lut(float c1p) {
  uint32_t p[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    p[k] = pack_bf16x2(__fmul_rn(code_value(2 * k), c1p), __fmul_rn(code_value(2 * k + 1), c1p));
  BlockLut t;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // p[2k] = (T[4k], T[4k+1]), p[2k+1] = (T[4k+2], T[4k+3])
    t.lo[k] = __builtin_amdgcn_perm(p[2 * k + 1], p[2 * k], 0x06040200u);
    t.hi[k] = __builtin_amdgcn_perm(p[2 * k + 1], p[2 * k], 0x07050301u);
  }
  return t;
}

// Four selectors (one 4-bit index per byte, element order) -> two bf16 pairs.
__device__ __forceinline__ void lut4(const BlockLut& t, uint32_t s, uint32_t& out01, uint32_t& out23) {
  // sa = s | ((s << 3) & 0x40404040) as one v_bitop3 (truth table 0xEA: (a & b) | c)
  uint32_t sa = __builtin_amdgcn_bitop3_b32(s << 3, 0x40404040u, s, 0xEA);
  uint32_t sb = sa ^ 0x48484848u;
  uint32_t lo = __builtin_amdgcn_perm(t.lo[1], t.lo[0], sa) & __builtin_amdgcn_perm(t.lo[3], t.lo[2], sb);
  uint32_t hi = __builtin_amdgcn_perm(t.hi[1], t.hi[0], sa) & __builtin_amdgcn_perm(t.hi[3], t.hi[2], sb);
  out01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  out23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// One packed dword (8 indices, element 2j in the high nibble of byte j) -> 8 bf16 in element
// order, as 4 dwords (o[0] = elements 0,1; ...).
__device__ __forceinline__ void dequant8(const BlockLut& t, uint32_t p, uint32_t o[4]) {
  uint32_t odd = p & 0x0F0F0F0Fu;            // elements 1,3,5,7
  uint32_t even = (p >> 4) & 0x0F0F0F0Fu;    // elements 0,2,4,6
  uint32_t s0 = __builtin_amdgcn_perm(odd, even, 0x05010400u);  // elements 0..3
  uint32_t s1 = __builtin_amdgcn_perm(odd, even, 0x07030602u);  // elements 4..7
  lut4(t, s0, o[0], o[1]);
  lut4(t, s1, o[2], o[3]);
}

// First dequantisation level for block b.
__device__ __forceinline__ float block_scale(const uint8_t* __restrict__ scale_q,
                                             const float* __restrict__ scale_c2, int64_t b) {
  return __fmul_rn(e4m3_decode(scale_q[b]), scale_c2[b / kGroup]);
}

// ------------------------------------------------------------------------------------------
// Wave-level reductions with DPP (row = 16 lanes) and readlane across rows.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// max over aligned groups of 8 lanes (all 8 lanes receive the result)
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));   // row_half_mirror
  return v;
}
// max over the whole wave (all lanes receive the result)
__device__ __forceinline__ float wave_max(float v) {
  v = max8(v);
  v = fmaxf(v, dpp_f<0x140>(v));   // row_mirror: combines the two halves of a row
  float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------------------------------
// LDS-DMA plumbing (buffer loads that write LDS directly: lane i's 16 bytes land at M0 + 16 i).
typedef __attribute__((address_space(3))) void lds_void;
constexpr int kRsrcFlags = 0x00020000;         // raw buffer, 32-bit data format
constexpr uint32_t kOutOfRange = 0x80000000u;  // a buffer offset past every record count used here

// s_waitcnt on the vector-memory counter alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier after the wave's LDS accesses complete. Written as inline asm so that the
// compiler does not add a wait for every LDS-DMA load in flight (it cannot tell that those target
// stages nobody reads before the next barrier); code that needs a DMA landed waits for it with
// wait_vmcnt before calling this.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace nf4
