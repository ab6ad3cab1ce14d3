// Adapter merged into the dequantised base weight, in bf16 (gfx950).
//
// "QLoRA, explained", Quality loss at merge time: training saw W~, the dequantised weight, never the
// original one, so the merge that preserves the trained model is out = W~ + s B A, served in bf16
// (s = lora_alpha / r, as in the forward). Here: W~ exactly as the dequantisation kernels produce it,
// the rank-r product B A in fp32 on MFMA (bf16 products are exact, fp32 accumulation), then
// fl32(W~ + fl32(s * (B A))) rounded once to bf16, nearest even.
//
// A workgroup (4 waves) owns a strip of 128 columns (two blocks per row) and a range of 64-row
// tiles. The strip of A is staged once in LDS, transposed ([column][j]), so that an MFMA operand
// fragment (4 consecutive j of one column) is one 8-byte read. Per tile, wave w takes rows
// 16 w .. 16 w + 15:
//   * v_mfma_f32_16x16x16_bf16 forms the 16 x 128 block of B A with the A strip as the row side
//     and B as the column side (operand lanes: row or column lane % 16, j = 4 (lane / 16) .. +3;
//     result lanes: column lane % 16, rows 4 (lane / 16) + i), so a lane holds four consecutive
//     columns of one row of B A, and s times it is written to the wave's rows of an LDS tile with
//     16-byte writes;
//   * lane l then takes row l / 4 of those 16 and the 32 columns 32 (l % 4) .. +31 (half a block):
//     it dequantises them with the block's bf16 table, adds the update read back from LDS and
//     stores 64 contiguous bytes (the four lanes of a row write the strip's 256 bytes).
// Only the wave's own rows pass through its LDS rows, so no workgroup barrier is needed per tile.
// The next tile's packed bytes, scales and B fragments are loaded while a tile is processed.
#include "common.h"
#include "launch.h"

namespace nf4 {

constexpr int kMgCols = 128;     // columns per strip
constexpr int kMgRows = 64;      // rows per tile
constexpr int kMgPitch = kMgCols + 4;   // fp32 pitch of the update tile (rows shift by 4 banks)
constexpr int kMgStage = kMgCols + 8;   // bf16 pitch of the output staging rows (in the same LDS)
static_assert(16 * kMgStage * 2 <= 16 * kMgPitch * 4, "staging fits in a wave's update rows");

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

  // Lane l dequantises row l / 4 of the wave's 16 and columns 32 q .. +31, q = l % 4; in a last
  // half strip the lanes past it redo their neighbour's columns, and a wave whose rows lie past N
  // (rows come in 16s) redoes the last 16 rows, so that every load and store is unconditional
  // (they write identical bytes).
  const int rl = lane >> 2, q = lane & 3;
  const int64_t col = k0 + 32 * (32 * q < cols ? q : q - 2);
  auto first_row = [&](int64_t t) { return min(t * kMgRows + 16 * wave, g.N - 16); };
  // A tile's inputs for this lane, loaded one tile ahead into one of two register slots (raw
  // loaded values only, so issuing the loads never waits for them): the B fragments of the MFMA
  // (row first + lane % 16, j = 16 s + 4 (lane / 16) ..), the 16 packed bytes, the aligned word
  // holding the block's scale code (in range: the block count is a multiple of 16) and the
  // block's second-level constant.
  struct TileIn {
    s16x4 bf[NT];
    u32x4 p;
    uint32_t cw;
    float c2;
  };
  auto load_tile = [&](int64_t t, TileIn& in) {
    const int64_t n0 = first_row(t);
#pragma unroll
    for (int s = 0; s < NT; ++s)
      in.bf[s] = *reinterpret_cast<const s16x4*>(g.B + (n0 + (lane & 15)) * r + 16 * s + 4 * (lane >> 4));
    const int64_t n = n0 + rl;
    const int64_t b = n * kb + col / kBlock;
    in.p = *reinterpret_cast<const u32x4*>(g.packed + (n * g.K + col) / 2);
    in.cw = *reinterpret_cast<const uint32_t*>(g.scale_q + (b & ~int64_t(3)));
    in.c2 = g.scale_c2[b / kGroup];
  };
  auto process = [&](int64_t t, const TileIn& in, TileIn& nx, int64_t t_next) {
    const int64_t n0 = first_row(t);
    // ---- s B A for rows n0 .. n0 + 15, all 128 columns
    f32x4 acc[kMgCols / 16];
#pragma unroll
    for (int ct = 0; ct < kMgCols / 16; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NT; ++s) {
      const int jj = 16 * s + 4 * (lane >> 4);
#pragma unroll
      for (int ct = 0; ct < kMgCols / 16; ++ct) {
        const s16x4 af = *reinterpret_cast<const s16x4*>(at + (ct * 16 + (lane & 15)) * AP + jj);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(af, in.bf[s], acc[ct], 0, 0, 0);
      }
    }
    // acc[ct][i] = (B A)[row lane % 16][column 16 ct + 4 (lane / 16) + i]: four consecutive columns
#pragma unroll
    for (int ct = 0; ct < kMgCols / 16; ++ct)
      *reinterpret_cast<f32x4*>(urow + (lane & 15) * kMgPitch + ct * 16 + 4 * (lane >> 4)) =
          f32x4{__fmul_rn(g.scale, acc[ct][0]), __fmul_rn(g.scale, acc[ct][1]), __fmul_rn(g.scale, acc[ct][2]),
                __fmul_rn(g.scale, acc[ct][3])};

    // the next tile's loads go out between this tile's MFMA part and its dequantisation, so that a
    // wave waiting for room in the CU's vector-memory queue does so with half its tile still to do
    load_tile(t_next, nx);
    __builtin_amdgcn_sched_barrier(0);

    // ---- dequantise, add, round, store
    const int64_t n = n0 + rl;
    const int64_t b = n * kb + col / kBlock;
    const uint32_t code = in.cw >> ((uint32_t)(b & 3) * 8u);   // e4m3_decode reads bits 0 .. 6
    const BlockLut lut = make_lut(__fmul_rn(e4m3_decode(code), in.c2));
    const float* u = urow + rl * kMgPitch + (col - k0);
    u32x4 o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t d[4];
      dequant8(lut, in.p[i], d);   // values 8 i .. 8 i + 7 as 4 bf16 pairs
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
    // ---- coalesced stores through LDS: the results go into this wave's update rows (every lane
    // has read its update values, and a wave's LDS accesses complete in order) as bf16 rows of
    // kMgStage values, then store instruction i writes rows 4 i .. 4 i + 3, 16 bytes per lane and
    // the 256 bytes of a row from 16 consecutive lanes (lanes past a half strip repeat the last
    // 16 bytes of their row, identical writes)
    uint16_t* stg = reinterpret_cast<uint16_t*>(urow);
    u32x4* sdst = reinterpret_cast<u32x4*>(stg + rl * kMgStage + (col - k0));
#pragma unroll
    for (int i = 0; i < 4; ++i) sdst[i] = o[i];
    const int c16 = min(lane & 15, cols / 8 - 1);
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const u32x4*>(stg + (4 * i + (lane >> 4)) * kMgStage + 8 * c16);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(g.out + (n0 + 4 * i + (lane >> 4)) * g.K + k0 + 8 * c16) = v[i];
  };

  // tiles in pairs, so that each slot stays one register set; the next tile's loads go out
  // before the current tile's arithmetic (past the range they re-read the last tile)
  if (t_begin >= t_end) return;
  TileIn s0, s1;
  load_tile(t_begin, s0);
  int64_t t = t_begin;
  for (; t + 1 < t_end; t += 2) {
    process(t, s0, s1, t + 1);
    process(t + 1, s1, s0, min(t + 2, t_end - 1));
  }
  if (t < t_end) process(t, s0, s1, t);
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
