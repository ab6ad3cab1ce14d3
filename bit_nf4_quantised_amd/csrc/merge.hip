// Adapter merged into the dequantised base weight, in bf16 (gfx950).
//
// "QLoRA, explained", Quality loss at merge time: the adapter was trained against the dequantised
// weight W~, so the merge that keeps what was trained is out = W~ + s B A, served in bf16 (s =
// lora_alpha / r, as in the forward). Here: W~ exactly as the dequantisation kernels produce it,
// the rank-r product B A in fp32 on MFMA (bf16 products are exact, fp32 accumulation), then
// fl32(W~ + fl32(s * (B A))) rounded once to bf16, nearest even.
//
// A workgroup (4 waves) owns a strip of 128 columns (two blocks per row) and a range of 64-row
// tiles. The strip of A is staged once in LDS, transposed ([column][j]), so that an MFMA operand
// fragment (4 consecutive j of one column) is one 8-byte read. Per tile, wave w takes rows
// 16 w .. 16 w + 15:
//   * v_mfma_f32_16x16x16_bf16 forms the 16 x 128 block of B A (operand lanes: row or column
//     lane % 16, j = 4 (lane / 16) .. +3; result lanes: column lane % 16, rows 4 (lane / 16) + i),
//     and s times it is written to the wave's rows of an LDS tile;
//   * lane l then takes row l / 4 of those 16 and the 32 columns 32 (l % 4) .. +31 (half a block):
//     it dequantises them with the block's bf16 table, adds the update read back from LDS and
//     stores 64 contiguous bytes (the four lanes of a row write the strip's 256 bytes).
// Only the wave's own rows pass through its LDS rows, so no workgroup barrier is needed per tile.
#include "common.h"
#include "launch.h"

namespace nf4 {

constexpr int kMgCols = 128;     // columns per strip
constexpr int kMgRows = 64;      // rows per tile
constexpr int kMgPitch = kMgCols + 4;   // fp32 pitch of the update tile (rows shift by 4 banks)

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

struct MergeArgs {
  const uint8_t* packed;
  const uint8_t* scale_q;
  const float* scale_c2;
  int64_t N, K;
  const uint16_t* A;    // [r x K] bf16
  const uint16_t* B;    // [N x r] bf16
  int r;
  float scale;
  int row_chunks;       // workgroups per strip
  uint16_t* out;        // [N x K] bf16
};

template <int NT>   // r / 16: the A strip holds exactly r rows, so small ranks leave room for more
                    // workgroups per CU
__global__ __launch_bounds__(256) void qlora_merge_kernel(const MergeArgs g) {
  // A strip, [column][j], columns padded to r + 4 values so that the 16 columns of an MFMA
  // fragment read fall on distinct banks
  constexpr int AP = 16 * NT + 4;
  __shared__ __attribute__((aligned(16))) uint16_t at[kMgCols * AP];
  __shared__ __attribute__((aligned(16))) float ut[kMgRows * kMgPitch];    // s B A of one tile
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int strip = blockIdx.x / g.row_chunks, chunk = blockIdx.x % g.row_chunks;
  const int64_t k0 = (int64_t)strip * kMgCols;
  const int cols = (int)min((int64_t)kMgCols, g.K - k0);   // 128, or 64 for a last half strip
  constexpr int r = 16 * NT;

  // ---- A strip, transposed into LDS (columns past K as zeros)
  for (int idx = tid; idx < r * kMgCols; idx += 256) {
    const int j = idx / kMgCols, c = idx % kMgCols;
    at[c * AP + j] = c < cols ? g.A[(int64_t)j * g.K + k0 + c] : (uint16_t)0;
  }
  __syncthreads();

  const int64_t tiles = (g.N + kMgRows - 1) / kMgRows;
  const int64_t per_chunk = (tiles + g.row_chunks - 1) / g.row_chunks;
  const int64_t t_begin = chunk * per_chunk, t_end = min(tiles, t_begin + per_chunk);
  const int64_t kb = g.K / kBlock;
  float* urow = ut + (16 * wave) * kMgPitch;   // this wave's 16 rows of the update tile

  for (int64_t t = t_begin; t < t_end; ++t) {
    const int64_t n0 = t * kMgRows + 16 * wave;   // this wave's first row
    if (n0 >= g.N) continue;                      // rows come in multiples of 16

    // ---- s B A for rows n0 .. n0 + 15, all 128 columns
    f32x4 acc[kMgCols / 16];
#pragma unroll
    for (int ct = 0; ct < kMgCols / 16; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < r; j0 += 16) {
      const int jj = j0 + 4 * (lane >> 4);
      const s16x4 bf = *reinterpret_cast<const s16x4*>(g.B + (n0 + (lane & 15)) * r + jj);
#pragma unroll
      for (int ct = 0; ct < kMgCols / 16; ++ct) {
        const s16x4 af = *reinterpret_cast<const s16x4*>(at + (ct * 16 + (lane & 15)) * AP + jj);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bf, af, acc[ct], 0, 0, 0);
      }
    }
#pragma unroll
    for (int ct = 0; ct < kMgCols / 16; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        urow[(4 * (lane >> 4) + i) * kMgPitch + ct * 16 + (lane & 15)] = __fmul_rn(g.scale, acc[ct][i]);

    // ---- dequantise, add, round, store: row n0 + lane / 4, columns 32 (lane % 4) .. +31
    const int rl = lane >> 2, q = lane & 3;
    const int64_t n = n0 + rl;
    if (32 * q < cols) {
      const int64_t col = k0 + 32 * q;
      const int64_t b = n * kb + col / kBlock;
      const u32x4 p = *reinterpret_cast<const u32x4*>(g.packed + (n * g.K + col) / 2);
      const BlockLut lut = make_lut(block_scale(g.scale_q, g.scale_c2, b));
      const float* u = urow + rl * kMgPitch + 32 * q;
      u32x4 o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t d[4];
        dequant8(lut, p[i], d);   // values 8 i .. 8 i + 7 as 4 bf16 pairs
        const f32x4 u0 = *reinterpret_cast<const f32x4*>(u + 8 * i);
        const f32x4 u1 = *reinterpret_cast<const f32x4*>(u + 8 * i + 4);
        const float uu[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(d[e] << 16), hi = __uint_as_float(d[e] & 0xFFFF0000u);
          d[e] = pack_bf16x2(__fadd_rn(lo, uu[2 * e]), __fadd_rn(hi, uu[2 * e + 1]));
        }
        o[i] = u32x4{d[0], d[1], d[2], d[3]};
      }
      u32x4* dst = reinterpret_cast<u32x4*>(g.out + n * g.K + col);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = o[i];
    }
  }
}

hipError_t launch_merge(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2, int64_t N,
                        int64_t K, const uint16_t* A, const uint16_t* B, int r, float scale, uint16_t* out,
                        hipStream_t stream) {
  const int64_t strips = (K + kMgCols - 1) / kMgCols;
  const int64_t tiles = (N + kMgRows - 1) / kMgRows;
  int64_t chunks = (2048 + strips - 1) / strips;   // about 2048 workgroups in all
  if (chunks > tiles) chunks = tiles;
  if (chunks < 1) chunks = 1;
  MergeArgs g{packed, scale_q, scale_c2, N, K, A, B, r, scale, (int)chunks, out};
  const dim3 grid((unsigned)(strips * chunks)), block(256);
  switch (r / 16) {
    case 1: hipLaunchKernelGGL(qlora_merge_kernel<1>, grid, block, 0, stream, g); break;
    case 2: hipLaunchKernelGGL(qlora_merge_kernel<2>, grid, block, 0, stream, g); break;
    case 3: hipLaunchKernelGGL(qlora_merge_kernel<3>, grid, block, 0, stream, g); break;
    case 4: hipLaunchKernelGGL(qlora_merge_kernel<4>, grid, block, 0, stream, g); break;
    case 5: hipLaunchKernelGGL(qlora_merge_kernel<5>, grid, block, 0, stream, g); break;
    case 6: hipLaunchKernelGGL(qlora_merge_kernel<6>, grid, block, 0, stream, g); break;
    case 7: hipLaunchKernelGGL(qlora_merge_kernel<7>, grid, block, 0, stream, g); break;
    default: hipLaunchKernelGGL(qlora_merge_kernel<8>, grid, block, 0, stream, g); break;
  }
  return hipGetLastError();
}

}  // namespace nf4
