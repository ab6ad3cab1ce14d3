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
//   fast path, in bin units: y = fma(w, 16 rcp(c), 16) (rcp to 1 ulp; 16 rcp(c) is exact; one
//     rounding) is within 2^-18 of 16 w / c + 16, so y <= 32 + 2^-17 and its truncation to an
//     unsigned integer (negative and NaN values convert to 0) is a bin index in 0 .. 32. The 15
//     decision midpoints m of the codebook, binned on a grid of width 1/16 over [-1, 1], fall one
//     per bin at most and at least 1.6e-3 (0.0256 bin units) from any bin edge, so the bin gives
//     the count of midpoints below up to the one midpoint inside the bin, stored as
//     fl32(16 m + 16) (within 2^-19 of the exact value) and compared with y directly: that
//     decides as w / c against m whenever the two differ by more than 2^-18 + 2^-19 bin units. If
//     y lies within 2^-16 bin units (2^-20 of w / c) of the midpoint, or the block scale is below
//     2^-100 (rcp(c) could overflow), the value takes the slow path;
//   slow path: count the midpoints m_i with w > c * m_i in fp64, where the product of a 24-bit
//     scale and a <= 26-bit midpoint is exact.
struct BinEntry {
  float mid;       // the midpoint inside the bin, or +inf
  uint32_t base;   // number of midpoints below the bin's lower edge
};

__device__ __forceinline__ double mid64(int i) {
  return ((double)code_value(i) + (double)code_value(i + 1)) * 0.5;
}

// BF16IN: the input is bf16 (a merged weight being re-quantised); its values widen to fp32 exactly,
// so the codes and scales are those of the same values given as fp32.
template <bool BF16IN>
__global__ __launch_bounds__(256) void nf4_quantize_kernel(const void* __restrict__ w,
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
      else if (m < hi) mid = (float)(16.0 * m + 16.0);   // in bin units
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
    if (valid && BF16IN) {
      const u32x4 h = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(w) + blk * kBlock + (lane & 7) * 8));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(h[e] << 16);
        v[2 * e + 1] = __uint_as_float(h[e] & 0xFFFF0000u);
      }
    } else if (valid) {
      const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(w) + blk * kBlock + (lane & 7) * 8);
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
    const float inv16 = 16.f * __builtin_amdgcn_rcpf(amax);
    const bool tiny = amax < 0x1p-100f;
    uint32_t word = 0;
    float dmin = __builtin_inff();   // closest approach of y to a bin's midpoint, over the 8 values
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float y = fmaf(v[e], inv16, 16.f);
      const BinEntry be = tab[__float2uint_rz(y)];
      const uint32_t idx = be.base + (y > be.mid ? 1u : 0u);
      dmin = fminf(dmin, fabsf(y - be.mid));
      word |= idx << (8 * (e >> 1) + ((e & 1) ? 0 : 4));
    }
    const bool any_slow = tiny || dmin <= 0x1p-16f;
    if (__builtin_expect(__any(any_slow), 0)) {
      if (any_slow) {
        const double c = (double)amax;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float y = fmaf(v[e], inv16, 16.f);
          if (tiny || fabsf(y - tab[__float2uint_rz(y)].mid) <= 0x1p-16f) {
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
//   x = c1 * rcp(c2) is within a few 2^-24 of the ratio (relative), far less than half the gap
//   between neighbouring E4M3 values (at least 2^-5 relative), so truncating x to E4M3 gives the
//   code just below the ratio or, when the ratio sits within that distance of an E4M3 value, that
//   value's neighbour. Either way the nearest code is the truncation c or c + 1, and the sign of
//   c1 - c2 * m, m their midpoint, decides: one fused multiply-add forms the exact difference and
//   rounds it once, which keeps its sign and whether it is zero (a tie, to the even code) as long
//   as nothing underflows. A group maximum below 2^-60 takes the correctly rounded quotient and an
//   fp64 test instead (c2 * m is exact in fp64: 24 times at most 5 significant bits).
__device__ __forceinline__ uint32_t e4m3_code_of_ratio_exact(float c1, float c2) {
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

// The common case (group maximum c2 >= 2^-60), without branches. rc = rcp(c2), shared by the
// group. x = c1 * rc is within a few 2^-24 of the ratio; the stochastic-rounding conversion to
// E4M3 with zero random bits rounds it toward zero, giving the code c just below x (subnormal
// codes included). The midpoint of c and c + 1 is the mean of their two exact decodes (both are
// E4M3 values, so the sum and the halving are exact in fp32), and the sign of one fma decides,
// ties to the even code. c <= 0x38 since the ratio is at most 1, and the midpoint to 0x39
// (1.0625) is above every ratio. (The truncation done with integer bit operations instead took
// twice the instructions and gave the same codes on 12.8 M probed pairs around every code value
// and midpoint.)
__device__ __forceinline__ uint32_t e4m3_code_of_ratio_fast(float c1, float c2, float rc) {
  const float x = __fmul_rn(c1, rc);
  const uint32_t c = (uint32_t)__builtin_amdgcn_cvt_sr_fp8_f32(x, 0, 0, 0) & 0xFFu;
  const float m = (__builtin_amdgcn_cvt_f32_fp8((int)c, 0) + __builtin_amdgcn_cvt_f32_fp8((int)(c + 1u), 0)) * 0.5f;
  const float d = __builtin_fmaf(-c2, m, c1);
  return c + ((d > 0.f) | ((d == 0.f) & (c & 1u)));
}

__device__ __forceinline__ uint32_t e4m3_code_of_ratio(float c1, float c2) {
  if (c2 == 0.f) return 0;
  if (c2 < 0x1p-60f) return e4m3_code_of_ratio_exact(c1, c2);
  return e4m3_code_of_ratio_fast(c1, c2, __builtin_amdgcn_rcpf(c2));
}

// the four codes of a lane's scales against its group's c2 (wave-uniform), one byte each
__device__ __forceinline__ uint32_t e4m3_codes4(const float c[4], float c2) {
  uint32_t word = 0;
  if (c2 == 0.f) return 0;
  if (c2 < 0x1p-60f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) word |= e4m3_code_of_ratio_exact(c[i], c2) << (8 * i);
  } else {
    const float rc = __builtin_amdgcn_rcpf(c2);
#pragma unroll
    for (int i = 0; i < 4; ++i) word |= e4m3_code_of_ratio_fast(c[i], c2, rc) << (8 * i);
  }
  return word;
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
      const float cc[4] = {cur[0], cur[1], cur[2], cur[3]};
      *reinterpret_cast<uint32_t*>(scale_q + g * kGroup + lane * 4) = e4m3_codes4(cc, c2);
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

// Double quantisation of several weights' scales in one launch. The tensors' groups are numbered
// one after the other (group_begin[t] is tensor t's first); each wave encodes kDqRun consecutive
// groups, exactly as nf4_double_quant_kernel encodes a group. It issues the loads of all of them
// before it encodes any, so every wave keeps kDqRun KB in flight and a launch holds many short
// waves instead of few long ones (a wave that walked 28 groups with two in flight spent most of
// its time on the round trip of each). The wave finds its first group's tensor by bisection and
// steps to the next tensor when its run crosses into it (empty tensors are not in the batch).
constexpr int kDqRun = 4;
__global__ __launch_bounds__(256) void nf4_double_quant_many_kernel(const DqBatch b) {
  const int lane = threadIdx.x & 63;
  const int64_t wv = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t total = b.group_begin[b.count];
  const int64_t g0 = wv * kDqRun;
  if (g0 >= total) return;
  int t = 0, hi = b.count;   // group_begin[t] <= g0 < group_begin[t + 1]
  while (hi - t > 1) {
    const int mid = (t + hi) >> 1;
    if (g0 >= b.group_begin[mid]) t = mid;
    else hi = mid;
  }
  // scales of group gg of tensor tt (zeros past the tensor's end)
  auto load = [&](int tt, int64_t gg) {
    const float* absmax = b.absmax[tt];
    const int64_t nblocks = b.nblocks[tt];
    const int64_t lg = gg - b.group_begin[tt], first = lg * kGroup + lane * 4;
    if ((lg + 1) * kGroup <= nblocks) return *reinterpret_cast<const f32x4*>(absmax + first);
    f32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (first + i < nblocks) ? absmax[first + i] : 0.f;
    return v;
  };
  int tt[kDqRun];
  f32x4 v[kDqRun];
#pragma unroll
  for (int i = 0; i < kDqRun; ++i) {
    const int64_t g = g0 + i;
    if (g < total) {
      while (g >= b.group_begin[t + 1]) ++t;
      tt[i] = t;
      v[i] = load(t, g);
    }
  }
#pragma unroll
  for (int i = 0; i < kDqRun; ++i) {
    const int64_t g = g0 + i;
    if (g >= total) break;
    uint8_t* scale_q = b.scale_q[tt[i]];
    const int64_t nblocks = b.nblocks[tt[i]];
    const int64_t lg = g - b.group_begin[tt[i]], first = lg * kGroup + lane * 4;
    const f32x4 cur = v[i];
    const float c2 = wave_max(fmaxf(fmaxf(cur[0], cur[1]), fmaxf(cur[2], cur[3])));
    if ((lg + 1) * kGroup <= nblocks) {
      const float cc[4] = {cur[0], cur[1], cur[2], cur[3]};
      *reinterpret_cast<uint32_t*>(scale_q + first) = e4m3_codes4(cc, c2);
    } else {
      for (int k = 0; k < 4; ++k)
        if (first + k < nblocks) scale_q[first + k] = (uint8_t)e4m3_code_of_ratio(cur[k], c2);
    }
    if (lane == 0) b.scale_c2[tt[i]][lg] = c2;
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

static hipError_t launch_quantize_any(const void* w, bool bf16_in, int64_t numel, uint8_t* packed,
                                      float* absmax, hipStream_t stream) {
  const int64_t nblocks = numel / kBlock;
  if (nblocks == 0) return hipSuccess;
  const int64_t iters = (nblocks + 7) / 8;         // one wave iteration per 8 blocks
  const int grid = grid_for(iters, 4, 256 * 32);   // 4 waves per workgroup
  if (bf16_in)
    hipLaunchKernelGGL(nf4_quantize_kernel<true>, dim3(grid), dim3(256), 0, stream, w, nblocks,
                       reinterpret_cast<uint32_t*>(packed), absmax);
  else
    hipLaunchKernelGGL(nf4_quantize_kernel<false>, dim3(grid), dim3(256), 0, stream, w, nblocks,
                       reinterpret_cast<uint32_t*>(packed), absmax);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* w, int64_t numel, uint8_t* packed, float* absmax,
                           hipStream_t stream) {
  return launch_quantize_any(w, false, numel, packed, absmax, stream);
}

hipError_t launch_quantize_bf16(const uint16_t* w, int64_t numel, uint8_t* packed, float* absmax,
                                hipStream_t stream) {
  return launch_quantize_any(w, true, numel, packed, absmax, stream);
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

hipError_t launch_double_quant_many(const DqBatch& b, hipStream_t stream) {
  const int64_t groups = b.group_begin[b.count];
  if (groups == 0) return hipSuccess;
  const int64_t waves = (groups + kDqRun - 1) / kDqRun;
  hipLaunchKernelGGL(nf4_double_quant_many_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, b);
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
