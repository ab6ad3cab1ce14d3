// NF4 quantisation, double quantisation and standalone dequantisation kernels (gfx950).
//
//   nf4_quantize_kernel      "QLoRA, explained", Blockwise absmax quantisation / NormalFloat 4:
//                            per block of 64 the absmax and, per value, the nearest code index,
//                            packed two per byte.
//   nf4_double_quant_kernel  same page, Double quantisation: scales to E4M3 in groups of 256 with
//                            one fp32 constant (the group maximum) per group.
//   nf4_dequant_kernel       same page, The forward pass and gradients: two-level dequantisation
//                            to bf16 (c1' = fl32(e4m3 * c2), w~ = bf16(fl32(q[idx] * c1'))).
#include "common.h"
#include "launch.h"

namespace nf4 {

// ------------------------------------------------------------------------------------------
// Quantise. One wave handles 8 blocks per iteration: lane l covers 8 consecutive values of block
// (l / 8). The nearest-code decision must be exact (as if w / c were computed without rounding):
//   fast path: x = w * (1/c) is within 2^-22.9 of w / c. The 15 decision midpoints of the
//     codebook, binned on a grid of width 1/16 over [-1, 1], fall one per bin at most and at least
//     1.6e-3 from any bin edge, so the bin of x gives the count of midpoints below it up to the
//     one midpoint inside the bin, which is compared directly. If x lies within 2^-20 of that
//     midpoint, or the block scale is below 2^-100 (1/c could overflow), the value takes the
//     slow path;
//   slow path: count the midpoints m_i with w > c * m_i in fp64, where the product of a 24-bit
//     scale and a <= 26-bit midpoint is exact.
struct BinEntry {
  float mid;       // the midpoint inside the bin, or +inf
  uint32_t base;   // number of midpoints below the bin's lower edge
};

__device__ __forceinline__ double mid64(int i) {
  return ((double)code_value(i) + (double)code_value(i + 1)) * 0.5;
}

__global__ __launch_bounds__(256) void nf4_quantize_kernel(const float* __restrict__ w,
                                                           int64_t nblocks,
                                                           uint32_t* __restrict__ packed,
                                                           float* __restrict__ absmax) {
  __shared__ BinEntry tab[33];
  if (threadIdx.x < 33) {
    const double lo = threadIdx.x / 16.0 - 1.0, hi = (threadIdx.x + 1) / 16.0 - 1.0;
    uint32_t base = 0;
    float mid = __builtin_inff();
    for (int i = 0; i < 15; ++i) {
      double m = mid64(i);
      if (m < lo) ++base;
      else if (m < hi) mid = (float)m;
    }
    tab[threadIdx.x] = BinEntry{mid, base};
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const int64_t iters = (nblocks + 7) / 8;
  for (int64_t it = wave; it < iters; it += nwaves) {
    const int64_t blk = it * 8 + (lane >> 3);
    const bool valid = blk < nblocks;
    float v[8];
    if (valid) {
      const f32x4* src = reinterpret_cast<const f32x4*>(w + blk * kBlock + (lane & 7) * 8);
      f32x4 a = __builtin_nontemporal_load(src), b = __builtin_nontemporal_load(src + 1);
      v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
      v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    amax = max8(amax);
    const float inv = 1.0f / amax;
    const bool tiny = amax < 0x1p-100f;
    uint32_t word = 0, slow = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = v[e] * inv;
      const uint32_t bin = min(__float2uint_rz(fmaf(x, 16.f, 16.f)), 32u);
      const BinEntry be = tab[bin];
      const uint32_t idx = be.base + (x > be.mid ? 1u : 0u);
      if (fabsf(x - be.mid) <= 0x1p-20f || tiny) slow |= 1u << e;
      word |= idx << (8 * (e >> 1) + ((e & 1) ? 0 : 4));
    }
    if (__builtin_expect(__any(slow != 0), 0)) {
      if (slow) {
        const double c = (double)amax;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (slow & (1u << e)) {
            uint32_t idx = 0;
            for (int i = 0; i < 15; ++i) idx += ((double)v[e] > c * mid64(i)) ? 1u : 0u;
            const int sh = 8 * (e >> 1) + ((e & 1) ? 0 : 4);
            word = (word & ~(0xFu << sh)) | (idx << sh);
          }
        }
      }
    }
    if (amax == 0.f) word = 0x77777777u;  // all-zero block: every value takes the zero code
    if (valid) {
      __builtin_nontemporal_store(word, packed + blk * 8 + (lane & 7));
      if ((lane & 7) == 0) absmax[blk] = amax;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Double quantisation. One wave per group of 256 scales, 4 per lane; a wave walks groups with a
// stride of the grid and has the next group's scales in flight while it encodes the current one.
// c2 is the exact group maximum; the code is the E4M3 value in [0, 1] nearest to the exact ratio
// c1 / c2, ties to the even code:
//   x = fl32(c1 / c2) (correctly rounded) is within 2^-24 x of the ratio, far less than the gap
//   between neighbouring E4M3 values, so truncating x to E4M3 gives the code just below the ratio
//   or, when the ratio sits within that distance of an E4M3 value, that value's neighbour. Either
//   way the nearest code is one of the truncation c and c + 1, and the exact test c1 > c2 * m
//   against their midpoint m decides (exact in fp64: a 24-bit scale times a midpoint of at most 5
//   significant bits), with equality going to the even code.
__device__ __forceinline__ uint32_t e4m3_code_of_ratio(float c1, float c2) {
  if (c2 == 0.f) return 0;
  const float x = __fdiv_rn(c1, c2);   // in [0, 1]
  uint32_t c;
  if (x < 0x1p-6f) {
    c = (uint32_t)(x * 0x1p9f);          // subnormal codes m * 2^-9, m = 0..7 (exact scaling)
  } else {
    const uint32_t bits = __float_as_uint(x);
    c = ((((bits >> 23) & 0xFFu) - 120u) << 3) | ((bits >> 20) & 7u);   // exponent field e + 7
  }
  if (c >= 0x38u) return 0x38u;          // 1.0, the largest value a ratio in [0, 1] can take
  const double m = ((double)e4m3_decode(c) + (double)e4m3_decode(c + 1)) * 0.5;
  const double a = c1, b = (double)c2 * m;
  if (a > b) return c + 1;
  if (a == b) return (c & 1u) ? c + 1 : c;
  return c;
}

__global__ __launch_bounds__(256) void nf4_double_quant_kernel(const float* __restrict__ absmax,
                                                               int64_t nblocks,
                                                               uint8_t* __restrict__ scale_q,
                                                               float* __restrict__ scale_c2) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const int64_t ngroups = (nblocks + kGroup - 1) / kGroup;
  const int64_t full = nblocks / kGroup;   // groups without a ragged end
  // full groups: branch-free 16-byte loads, the next group's in flight
  auto load = [&](int64_t g) {
    return *reinterpret_cast<const f32x4*>(absmax + g * kGroup + lane * 4);
  };
  int64_t g = gw;
  if (g < full) {
    f32x4 cur = load(g);
    for (; g < full; g += nw) {
      const f32x4 nxt = load(min(g + nw, full - 1));
      const float c2 = wave_max(fmaxf(fmaxf(cur[0], cur[1]), fmaxf(cur[2], cur[3])));
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) word |= e4m3_code_of_ratio(cur[i], c2) << (8 * i);
      *reinterpret_cast<uint32_t*>(scale_q + g * kGroup + lane * 4) = word;
      if (lane == 0) scale_c2[g] = c2;
      cur = nxt;
    }
  }
  // the ragged last group, if any, by the wave whose turn it is
  if (full < ngroups && gw == full % nw) {
    const int64_t first = full * kGroup + lane * 4;
    float c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = (first + i < nblocks) ? absmax[first + i] : 0.f;
    const float c2 = wave_max(fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3])));
    for (int i = 0; i < 4; ++i)
      if (first + i < nblocks) scale_q[first + i] = (uint8_t)e4m3_code_of_ratio(c[i], c2);
    if (lane == 0) scale_c2[full] = c2;
  }
}

// ------------------------------------------------------------------------------------------
// Dequantise. A wave takes 64 consecutive blocks, lane l block l: it loads the 32 packed bytes,
// builds the block's 16-entry bf16 table and expands its 8 dwords into 8 pieces of 8 bf16 (16 bytes
// each, 128 bytes per lane). The pieces go through a wave-private LDS region so that every store
// instruction writes 1 KB of contiguous output (lane l: bytes 16 l + 1024 i of the wave's 8 KB);
// piece j of lane l sits at slot 8 l + (j ^ (l % 8)), which keeps both the writes and the reads of
// 8 consecutive lanes on distinct banks. Every wave handles exactly one group of 64 blocks: with a
// capped, persistent grid the group count rarely divides evenly, and the waves that take one
// more group than the rest set the kernel's duration.
constexpr int kDqWaves = 4;

__global__ __launch_bounds__(kDqWaves * 64) void nf4_dequant_kernel(const uint8_t* __restrict__ packed,
                                                                    const uint8_t* __restrict__ scale_q,
                                                                    const float* __restrict__ scale_c2,
                                                                    int64_t nblocks, u32x4* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) u32x4 stage[kDqWaves][64 * 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u32x4* st = stage[wave];
  const int64_t grp = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t groups = (nblocks + 63) / 64;
  if (grp >= groups) return;

  // branch-free loads: blocks past the end re-read the last block
  const int64_t b = min(grp * 64 + lane, nblocks - 1);
  const u32x4* src = reinterpret_cast<const u32x4*>(packed + b * 32);
  const u32x4 p0 = __builtin_nontemporal_load(src);
  const u32x4 p1 = __builtin_nontemporal_load(src + 1);
  const uint32_t code = scale_q[b];
  const float c2 = scale_c2[b / kGroup];

  const BlockLut t = make_lut(__fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)code, 0), c2));
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t d[4];
    dequant8(t, j < 4 ? p0[j] : p1[j - 4], d);
    st[lane * 8 + (j ^ (lane & 7))] = u32x4{d[0], d[1], d[2], d[3]};
  }
  // read back and store coalesced: instruction i covers output bytes 1024 i .. +1023 of the
  // group, i.e. piece lane % 8 of block 8 i + lane / 8. Slots of blocks past the end hold the
  // last block's values (its packed bytes were re-read), so storing them over the last block
  // writes identical bytes and every store stays unconditional.
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int lb = 8 * i + (lane >> 3), pj = lane & 7;
    v[i] = st[lb * 8 + (pj ^ (lb & 7))];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t bo = min(grp * 64 + 8 * i + (lane >> 3), nblocks - 1);
    __builtin_nontemporal_store(v[i], out + bo * 8 + (lane & 7));
  }
}

// ------------------------------------------------------------------------------------------
static int grid_for(int64_t work_items, int per_block, int max_blocks) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > max_blocks) g = max_blocks;
  return (int)g;
}

hipError_t launch_quantize(const float* w, int64_t numel, uint8_t* packed, float* absmax,
                           hipStream_t stream) {
  const int64_t nblocks = numel / kBlock;
  if (nblocks == 0) return hipSuccess;
  const int64_t iters = (nblocks + 7) / 8;         // one wave iteration per 8 blocks
  const int grid = grid_for(iters, 4, 256 * 32);   // 4 waves per workgroup
  hipLaunchKernelGGL(nf4_quantize_kernel, dim3(grid), dim3(256), 0, stream, w, nblocks,
                     reinterpret_cast<uint32_t*>(packed), absmax);
  return hipGetLastError();
}

hipError_t launch_double_quant(const float* absmax, int64_t nblocks, uint8_t* scale_q,
                               float* scale_c2, hipStream_t stream) {
  if (nblocks == 0) return hipSuccess;
  const int64_t ngroups = (nblocks + kGroup - 1) / kGroup;
  const int grid = grid_for(ngroups, 4, 256 * 8);   // 4 waves per workgroup, one group each
  hipLaunchKernelGGL(nf4_double_quant_kernel, dim3(grid), dim3(256), 0, stream, absmax, nblocks,
                     scale_q, scale_c2);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                          int64_t numel, uint16_t* out, hipStream_t stream) {
  const int64_t nblocks = numel / kBlock;
  if (nblocks == 0) return hipSuccess;
  const int64_t groups = (nblocks + 63) / 64;      // one wave per 64 blocks
  const int grid = (int)((groups + kDqWaves - 1) / kDqWaves);
  hipLaunchKernelGGL(nf4_dequant_kernel, dim3(grid), dim3(kDqWaves * 64), 0, stream, packed, scale_q,
                     scale_c2, nblocks, reinterpret_cast<u32x4*>(out));
  return hipGetLastError();
}

}  // namespace nf4
