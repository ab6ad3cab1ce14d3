// Codebook and blocksize variants of the 4-bit format, and scales without double quantisation
// (gfx950).
//
// "QLoRA, explained", A toy run (NF4 beside an INT4 grid of 15 levels k/7 and E2M1 FP4 rescaled to
// [-1, 1]), its blocksize discussion (16 to 4096 values per absmax) and Double quantisation (whose
// baseline keeps one fp32 absmax per block):
//   q4_quantize_kernel<B>       blockwise absmax over blocks of B values and, per value, the exact
//                               nearest code of w / c in an ascending codebook of 15 or 16 values,
//                               two indices per byte (element 2j in the high nibble of byte j);
//   q4_dequant_kernel<L, DQ>    bf16(fl32(q[idx] * s)), s = the fp32 absmax itself, or
//                               fl32(e4m3 * c2) when the scales are double quantised.
//
// Exact nearest code for any such codebook: x = w * rcp(c) (rcp to 1 ulp) is within 1.5 * 2^-23 of
// w / c. A table of 256 bins of width 1/128 over [-1, 1], built once on the host from the codebook
// and copied into LDS by each workgroup, holds per bin the number of decision midpoints below it and the
// midpoint inside it (at most one: the codebooks' midpoints are at least 0.04 apart). Then idx = base + (x > mid) is the
// exact count of midpoints below x, and it equals the count below w / c unless x lies within 2^-20
// of the bin's midpoint or of one of its edges (or the scale is below 2^-100): such values count
// the midpoints m with w > c * m in fp64, where the product of a 24-bit scale and a midpoint of at
// most 26 bits is exact. A value exactly on a midpoint takes the lower index; an all-zero block
// takes the codebook's zero; w = -c and w = +c take the end codes -1 and +1 directly.
#include <math.h>
#include <string.h>

#include "common.h"
#include "launch.h"

namespace nf4 {

struct Q4Book {
  float q[16];       // ascending; entry 15 repeats the last code when there are 15
  int count;         // 15 or 16
  int zero_index;    // the code that is exactly 0
};

// ------------------------------------------------------------------------------------------
// Quantise: a workgroup of 256 threads takes 4096 consecutive values, a thread 16 of them (four
// 16-byte loads), so a block of B values spans B / 16 consecutive threads.
constexpr int kQBins = 256;
constexpr float kQMargin = 0x1p-20f;

struct QBin {
  float mid;         // the midpoint inside the bin, or +inf
  uint32_t base;     // midpoints below the bin's lower edge
};

struct QBinTable {
  QBin bin[kQBins];
};

// Maximum over the B / 16 threads of a block: a butterfly within the wave, then (B > 1024) the
// wave maxima through LDS.
template <int B>
__device__ __forceinline__ float block_max(float v, float* wmax) {
  constexpr int seg = B / 16;
  constexpr int inwave = seg < 64 ? seg : 64;
#pragma unroll
  for (int o = 1; o < inwave; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  if constexpr (seg > 64) {
    constexpr int wpb = seg / 64;
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) wmax[wave] = v;
    __syncthreads();
    const int first = wave & ~(wpb - 1);
    float r = wmax[first];
#pragma unroll
    for (int k = 1; k < wpb; ++k) r = fmaxf(r, wmax[first + k]);
    v = r;
  }
  return v;
}

__device__ uint32_t exact_index(float w, float c, const Q4Book& cb) {
  if (c == 0.f) return (uint32_t)cb.zero_index;
  const double wd = w, cd = c;
  uint32_t idx = 0;
  for (int i = 0; i + 1 < cb.count; ++i)
    idx += wd > cd * (((double)cb.q[i] + (double)cb.q[i + 1]) * 0.5) ? 1u : 0u;
  return idx;
}

template <int B>
__global__ __launch_bounds__(256) void q4_quantize_kernel(const f32x4* __restrict__ w, int64_t numel,
                                                          const Q4Book cb, const QBinTable table,
                                                          u32x2* __restrict__ packed,
                                                          float* __restrict__ absmax) {
  __shared__ QBin bins[kQBins];
  __shared__ float wmax[4];
  bins[threadIdx.x] = table.bin[threadIdx.x];
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 16;
  const bool valid = e0 < numel;
  const int64_t ec = valid ? e0 : numel - 16;      // blocks past the end re-read the last values
  f32x4 x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = w[ec / 4 + i];
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) a = fmaxf(a, fabsf(x[i][k]));
  __syncthreads();                                  // the bin table is complete
  const float c = block_max<B>(a, wmax);
  if (valid && (threadIdx.x & (B / 16 - 1)) == 0) absmax[e0 / B] = c;

  const bool tiny = c < 0x1p-100f;                  // includes an all-zero block
  const float inv = tiny ? 0.f : __builtin_amdgcn_rcpf(c);
  uint32_t idx[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const float val = x[v / 4][v % 4];
    const float xv = __fmul_rn(val, inv);
    int bi = (int)__fmul_rn(__fadd_rn(xv, 1.0f), 128.0f);
    bi = bi < 0 ? 0 : (bi > kQBins - 1 ? kQBins - 1 : bi);
    const QBin e = bins[bi];
    const float lo = __fadd_rn(-1.0f, (float)bi * (1.0f / 128.0f));   // exact
    const float hi = __fadd_rn(lo, 1.0f / 128.0f);                     // exact
    // w = +-c is the last or first code exactly (every codebook here ends at -1 and +1); without
    // this, each block's own maximum would sit on the last bin's edge and send a lane of almost
    // every wave down the fp64 path
    const bool at_end = fabsf(val) == c;
    const bool slow = tiny || (!at_end && (fabsf(xv - e.mid) < kQMargin || xv - lo < kQMargin ||
                                           hi - xv < kQMargin));
    const uint32_t fast = at_end ? (val > 0.f ? (uint32_t)cb.count - 1u : 0u)
                                 : e.base + (xv > e.mid ? 1u : 0u);
    idx[v] = slow ? exact_index(val, c, cb) : fast;
  }
  u32x2 out = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j / 4] |= ((idx[2 * j] << 4) | idx[2 * j + 1]) << (8 * (j % 4));
  if (valid) packed[e0 / 16] = out;
}

// ------------------------------------------------------------------------------------------
// Dequantise: as the NF4 kernel, a wave takes 64 units of 64 consecutive values, a lane one unit
// (two 16-byte loads of packed indices), builds the bf16 table of each block its unit touches
// (L = 4 blocks at B = 16, 2 at B = 32, else 1) and expands its eight packed dwords by byte
// permutes; the results go through a swizzled wave-private LDS region so that each store
// instruction writes 1 KB of contiguous output.
constexpr int kQdWaves = 4;

template <int L, bool kDQ>
__global__ __launch_bounds__(kQdWaves * 64) void q4_dequant_kernel(const uint8_t* __restrict__ packed,
                                                                   const float* __restrict__ absmax,
                                                                   const uint8_t* __restrict__ scale_q,
                                                                   const float* __restrict__ scale_c2,
                                                                   int64_t units, int unit_shift,
                                                                   const Q4Book cb, u32x4* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) u32x4 stage[kQdWaves][64 * 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u32x4* st = stage[wave];
  const int64_t grp = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t groups = (units + 63) / 64;
  if (grp >= groups) return;

  // branch-free loads: units past the end re-read the last unit
  const int64_t u = min(grp * 64 + lane, units - 1);
  const u32x4* src = reinterpret_cast<const u32x4*>(packed + u * 32);
  const u32x4 p0 = __builtin_nontemporal_load(src);
  const u32x4 p1 = __builtin_nontemporal_load(src + 1);
  BlockLut t[L];
#pragma unroll
  for (int l = 0; l < L; ++l) {
    const int64_t b = L == 1 ? (u >> unit_shift) : u * L + l;
    const float s = kDQ ? __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)scale_q[b], 0), scale_c2[b / kGroup])
                        : absmax[b];
    t[l] = make_lut(s, cb.q);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t d[4];
    dequant8(t[j * L / 8], j < 4 ? p0[j] : p1[j - 4], d);
    st[lane * 8 + (j ^ (lane & 7))] = u32x4{d[0], d[1], d[2], d[3]};
  }
  // instruction i stores output bytes 1024 i .. +1023 of the wave's units: piece lane % 8 of unit
  // 8 i + lane / 8 (slots of units past the end hold the last unit's values, so those stores
  // write identical bytes)
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int lu = 8 * i + (lane >> 3), pj = lane & 7;
    v[i] = st[lu * 8 + (pj ^ (lu & 7))];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t uo = min(grp * 64 + 8 * i + (lane >> 3), units - 1);
    __builtin_nontemporal_store(v[i], out + uo * 8 + (lane & 7));
  }
}

// ------------------------------------------------------------------------------------------
// The codebooks, built from their definitions: NF4 (the 16 codes above), E2M1 FP4 magnitudes
// {0, 0.5, 1, 1.5, 2, 3, 4, 6} / 6 with both signs (one zero, 15 values), and the symmetric INT4
// grid k / 7, k = -7..7 (15 values). Each value is the fp32 rounding of the exact quotient.
static bool make_book(int id, Q4Book& b) {
  static const uint32_t nf4_bits[16] = {NF4_CODE_BITS};
  if (id == 0) {
    for (int i = 0; i < 16; ++i) memcpy(&b.q[i], &nf4_bits[i], 4);
    b.count = 16;
    b.zero_index = 7;
  } else if (id == 1) {
    static const double mags[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    for (int i = 0; i < 7; ++i) b.q[i] = (float)(-mags[7 - i] / 6.0);
    for (int i = 0; i < 8; ++i) b.q[7 + i] = (float)(mags[i] / 6.0);
    b.q[15] = b.q[14];
    b.count = 15;
    b.zero_index = 7;
  } else if (id == 2) {
    for (int k = -7; k <= 7; ++k) b.q[k + 7] = (float)(k / 7.0);
    b.q[15] = b.q[14];
    b.count = 15;
    b.zero_index = 7;
  } else {
    return false;
  }
  // the quantiser maps w = -c and w = +c straight to the end codes
  if (b.q[0] != -1.0f || b.q[b.count - 1] != 1.0f) return false;
  // the bin table holds one midpoint per 1/128 bin at most
  for (int i = 0; i + 2 < b.count; ++i) {
    const double m0 = ((double)b.q[i] + b.q[i + 1]) * 0.5, m1 = ((double)b.q[i + 1] + b.q[i + 2]) * 0.5;
    if (m1 - m0 <= 1.0 / 128.0) return false;
  }
  return true;
}

bool codes_of(int book, Codes& out) {
  Q4Book b;
  if (!make_book(book, b)) return false;
  for (int i = 0; i < 16; ++i) out.v[i] = b.q[i];
  return true;
}

bool q4_codebook(int id, float out[16], int* count) {
  Q4Book b;
  if (!make_book(id, b)) return false;
  for (int i = 0; i < 16; ++i) out[i] = b.q[i];
  *count = b.count;
  return true;
}

// The bin table of a codebook: per bin [lo, hi) of width 1/128, the midpoints below lo and the one
// in [lo, hi) (each midpoint the exact fp64 mean of two fp32 codes, stored rounded to fp32; the
// kernel's 2^-20 margin around it covers that rounding).
static void make_bins(const Q4Book& cb, QBinTable& t) {
  for (int b = 0; b < kQBins; ++b) {
    const double lo = -1.0 + b / 128.0, hi = -1.0 + (b + 1) / 128.0;
    uint32_t base = 0;
    float mid = __builtin_huge_valf();
    for (int i = 0; i + 1 < cb.count; ++i) {
      const double m = ((double)cb.q[i] + (double)cb.q[i + 1]) * 0.5;
      if (m < lo) ++base;
      else if (m < hi) mid = (float)m;
    }
    t.bin[b] = QBin{mid, base};
  }
}

hipError_t launch_q4_quantize(const float* w, int64_t numel, int book, int blocksize, uint8_t* packed,
                              float* absmax, hipStream_t stream) {
  if (numel == 0) return hipSuccess;
  Q4Book cb;
  if (!make_book(book, cb)) return hipErrorInvalidValue;
  // built once, on first use, by a thread-safe static initialiser; constant afterwards
  struct Tables {
    QBinTable t[3];
    Tables() {
      for (int id = 0; id < 3; ++id) {
        Q4Book b;
        make_book(id, b);
        make_bins(b, t[id]);
      }
    }
  };
  static const Tables tables;
  const QBinTable& tb = tables.t[book];
  const dim3 grid((unsigned)((numel + 4095) / 4096)), block(256);
  const f32x4* src = reinterpret_cast<const f32x4*>(w);
  u32x2* dst = reinterpret_cast<u32x2*>(packed);
  switch (blocksize) {
    case 16: hipLaunchKernelGGL(q4_quantize_kernel<16>, grid, block, 0, stream, src, numel, cb, tb, dst, absmax); break;
    case 32: hipLaunchKernelGGL(q4_quantize_kernel<32>, grid, block, 0, stream, src, numel, cb, tb, dst, absmax); break;
    case 64: hipLaunchKernelGGL(q4_quantize_kernel<64>, grid, block, 0, stream, src, numel, cb, tb, dst, absmax); break;
    case 128: hipLaunchKernelGGL(q4_quantize_kernel<128>, grid, block, 0, stream, src, numel, cb, tb, dst, absmax); break;
    case 256: hipLaunchKernelGGL(q4_quantize_kernel<256>, grid, block, 0, stream, src, numel, cb, tb, dst, absmax); break;
    case 512: hipLaunchKernelGGL(q4_quantize_kernel<512>, grid, block, 0, stream, src, numel, cb, tb, dst, absmax); break;
    case 1024: hipLaunchKernelGGL(q4_quantize_kernel<1024>, grid, block, 0, stream, src, numel, cb, tb, dst, absmax); break;
    case 2048: hipLaunchKernelGGL(q4_quantize_kernel<2048>, grid, block, 0, stream, src, numel, cb, tb, dst, absmax); break;
    case 4096: hipLaunchKernelGGL(q4_quantize_kernel<4096>, grid, block, 0, stream, src, numel, cb, tb, dst, absmax); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_q4_dequant(const uint8_t* packed, const float* absmax, const uint8_t* scale_q,
                             const float* scale_c2, int64_t numel, int book, int blocksize, uint16_t* out,
                             hipStream_t stream) {
  if (numel == 0) return hipSuccess;
  Q4Book cb;
  if (!make_book(book, cb)) return hipErrorInvalidValue;
  const int64_t units = numel / 64;
  const dim3 grid((unsigned)(((units + 63) / 64 + kQdWaves - 1) / kQdWaves)), block(kQdWaves * 64);
  int shift = 0;
  while ((64 << shift) < blocksize) ++shift;
  u32x4* dst = reinterpret_cast<u32x4*>(out);
  const bool dq = absmax == nullptr;
  if (blocksize == 16) {
    if (dq) hipLaunchKernelGGL((q4_dequant_kernel<4, true>), grid, block, 0, stream, packed, absmax, scale_q, scale_c2, units, 0, cb, dst);
    else hipLaunchKernelGGL((q4_dequant_kernel<4, false>), grid, block, 0, stream, packed, absmax, scale_q, scale_c2, units, 0, cb, dst);
  } else if (blocksize == 32) {
    if (dq) hipLaunchKernelGGL((q4_dequant_kernel<2, true>), grid, block, 0, stream, packed, absmax, scale_q, scale_c2, units, 0, cb, dst);
    else hipLaunchKernelGGL((q4_dequant_kernel<2, false>), grid, block, 0, stream, packed, absmax, scale_q, scale_c2, units, 0, cb, dst);
  } else {
    if (dq) hipLaunchKernelGGL((q4_dequant_kernel<1, true>), grid, block, 0, stream, packed, absmax, scale_q, scale_c2, units, shift, cb, dst);
    else hipLaunchKernelGGL((q4_dequant_kernel<1, false>), grid, block, 0, stream, packed, absmax, scale_q, scale_c2, units, shift, cb, dst);
  }
  return hipGetLastError();
}

}  // namespace nf4
