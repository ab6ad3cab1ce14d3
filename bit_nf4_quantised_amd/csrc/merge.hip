// Adapter merged into the dequantised base weight, in bf16 (gfx950).
//
// "QLoRA, explained", Quality loss at merge time: training saw W~, the dequantised weight, never the
// original one, so the merge that preserves the trained model is out = W~ + s B A, served in bf16
// (s = lora_alpha / r, as in the forward). The result is the exact value W~ + s B A rounded once to
// bf16 (nearest, ties to even), W~ exactly as the dequantisation kernels produce it.
//
// Exactness. The fast path forms B A on MFMA in fp32 (the bf16 products are exact; only the
// accumulation rounds, and the matrix unit's is not a correctly rounded sum), then
// x = fl32(W~ + s (B A)) with one fma. Against the exact value X*,
//   |x - X*| <= ulp(x) / 2 + |s| E,   E = 2 (r + 1) 2^-24 sum_j |B[n][j] A[j][k]|
// (E bounds any summation of the r products with faithful roundings, with a factor 2 to spare),
// and sum_j |B[n][j] A[j][k]| <= |B[n]|_2 |A[:,k]|_2 (Cauchy-Schwarz), which the kernel bounds per
// lane by the row's norm times the largest column norm among the lane's 32 columns. x and the
// bf16 rounding tie of its cell, t = (x & 0xFFFF0000) | 0x8000, lie on one fp32 grid, so x != t
// means |x - t| >= ulp(x); then |x - t| > 2 |s| E puts X* strictly on x's side of t and
// bf16(x) = bf16(X*). The test costs four VALU operations per value. Values that fail it (a few
// per thousand at LoRA scales, mostly where W~ = 0 and the adapter term alone is rounded) are
// recomputed in the same tile: the wave lists them in LDS with their W~, then one lane per listed
// value forms the products exactly in fp32, sums them in float64 in j order, adds s times the sum
// to W~ with one fma and rounds once to bf16, writing the staging rows before the tile's global
// store. The float64 sum is exact whenever the products' exponents span less than 2^30, which
// bf16 factors of similar magnitude always meet. The recomputation reads only LDS (the B rows of
// the tile are staged there from the MFMA fragments), so the tile loop never waits on memory for it.
//
// Layout. A workgroup (4 waves) owns a strip of 128 columns (two blocks per row) and a range of
// 64-row tiles. The strip of A is staged once in LDS, transposed ([column][j]), so that an MFMA
// operand fragment (4 consecutive j of one column) is one 8-byte read. Per tile, wave w takes rows
// 16 w .. 16 w + 15:
//   * v_mfma_f32_16x16x16_bf16 forms the 16 x 128 block of B A with the A strip as the row side
//     and B as the column side (operand lanes: row or column lane % 16, j = 4 (lane / 16) .. +3;
//     result lanes: column lane % 16, rows 4 (lane / 16) + i), so a lane holds four consecutive
//     columns of one row of B A, written to the wave's rows of an LDS tile with 16-byte writes;
//     the row's squared norm goes to the tile row's padding;
//   * lane l then takes row l / 4 of those 16 and the 32 columns 32 (l % 4) .. +31 (half a block):
//     it looks its codes up in the block's table as fp32 values, adds s times the product read
//     back from LDS, tests for a near tie, rounds and stores 64 contiguous bytes through LDS (the
//     four lanes of a row write the strip's 256 bytes).
// Only the wave's own rows pass through its LDS rows, so no workgroup barrier is needed per tile.
// The next tile's packed bytes, scales and B fragments are loaded while a tile is processed.
#include "common.h"
#include "launch.h"

namespace nf4 {

constexpr int kMgCols = 128;     // columns per strip
constexpr int kMgRows = 64;      // rows per tile
constexpr int kMgPitch = kMgCols + 4;   // fp32 pitch of the product tile (rows shift by 4 banks);
                                        // column kMgCols holds the row's squared norm of B
constexpr int kMgStage = kMgCols + 8;   // bf16 pitch of the output staging rows (in the same LDS)
// a wave's LDS rows: the staging rows first, then the list of near-tie values of the tile
constexpr int kMgListOff = 16 * kMgStage * 2;                 // bytes
constexpr int kMgListCap = (16 * kMgPitch * 4 - kMgListOff) / 4;
static_assert(kMgListCap >= 128, "room for two rounds of listed values");

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
  float tie_coef;       // 4 |s| (r + 1) 2^-24, rounded up: the near-tie radius per unit of the bound
  float tie_floor;      // smallest radius (covers products an accumulator might flush to zero)
  int row_chunks;       // workgroups per strip
  uint16_t* out;        // [N x K] bf16
  Codes codes;          // the values the 4-bit indices select
};

__device__ __forceinline__ float bf16_val(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round a float64 value to bf16 once (nearest, ties to even). Magnitudes below 2^-126 (the bf16
// subnormal range) go through fp32 first.
__device__ __forceinline__ uint32_t bf16_from_f64(double x) {
  const uint64_t bits = (uint64_t)__double_as_longlong(x);
  const uint64_t sign = bits >> 63, mag = bits & 0x7FFFFFFFFFFFFFFFull;
  if (mag < (uint64_t(1023 - 126) << 52)) return pack_bf16x2((float)x, 0.f) & 0xFFFFu;
  // keep 7 of the 52 fraction bits: add just under half of the dropped range, plus the kept
  // field's lowest bit (ties to even); a carry moves into the exponent as it should
  const uint64_t t = (mag + ((uint64_t(1) << 44) - 1) + ((mag >> 45) & 1)) >> 45;   // exponent:7 bits
  const uint64_t e = t >> 7;                                                         // biased by 1023
  if (e >= 1023 + 128) return (uint32_t)((sign << 15) | 0x7F80u);                    // overflow: inf
  return (uint32_t)((sign << 15) | (t - (uint64_t(1023 - 127) << 7)));
}

// Byte-plane table lookup (as lut4) of the four selectors in s, one 4-bit index per byte; returns
// the two planes (lo: low bytes of the four bf16 values, hi: their high bytes).
__device__ __forceinline__ void lut4_planes(const BlockLut& t, uint32_t s, uint32_t& lo, uint32_t& hi) {
  const uint32_t sa = __builtin_amdgcn_bitop3_b32(s << 3, 0x40404040u, s, 0xEA);
  const uint32_t sb = sa ^ 0x48484848u;
  lo = __builtin_amdgcn_perm(t.lo[1], t.lo[0], sa) & __builtin_amdgcn_perm(t.lo[3], t.lo[2], sb);
  hi = __builtin_amdgcn_perm(t.hi[1], t.hi[0], sa) & __builtin_amdgcn_perm(t.hi[3], t.hi[2], sb);
}

// The four table values of the selectors in s as fp32 bit patterns: one v_perm per value places
// its two bytes in the upper half of a word (selector bytes: 0x0C gives zero; 0..3 the bytes of lo,
// 4..7 those of hi).
__device__ __forceinline__ void lut4_f32(const BlockLut& t, uint32_t s, uint32_t o[4]) {
  uint32_t lo, hi;
  lut4_planes(t, s, lo, hi);
  o[0] = __builtin_amdgcn_perm(hi, lo, 0x04000C0Cu);
  o[1] = __builtin_amdgcn_perm(hi, lo, 0x05010C0Cu);
  o[2] = __builtin_amdgcn_perm(hi, lo, 0x06020C0Cu);
  o[3] = __builtin_amdgcn_perm(hi, lo, 0x07030C0Cu);
}

template <int NT, bool NTSTORE>   // r / 16 (the A strip holds exactly r rows); nontemporal stores
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 4 : 1)))
void qlora_merge_kernel(const MergeArgs g) {
  // A strip, [column][j], columns padded to r + 4 values so that the 16 columns of an MFMA
  // fragment read fall on distinct banks
  constexpr int r = 16 * NT;
  constexpr int AP = r + 4;
  __shared__ __attribute__((aligned(16))) uint16_t at[kMgCols * AP];
  __shared__ __attribute__((aligned(16))) float ut[kMgRows * kMgPitch];    // B A of one tile
  __shared__ __attribute__((aligned(16))) uint16_t brow[4][16 * r];       // B rows of the tile
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int strip = blockIdx.x / g.row_chunks, chunk = blockIdx.x % g.row_chunks;
  const int64_t k0 = (int64_t)strip * kMgCols;
  const int cols = (int)min((int64_t)kMgCols, g.K - k0);   // 128, or 64 for a last half strip

  // ---- A strip, transposed into LDS (columns past K as zeros), and its column norms |A[:,k]|_2
  for (int idx = tid; idx < r * kMgCols; idx += 256) {
    const int j = idx / kMgCols, c = idx % kMgCols;
    at[c * AP + j] = c < cols ? g.A[(int64_t)j * g.K + k0 + c] : (uint16_t)0;
  }
  __syncthreads();
  float* colnorm = ut;   // in the product tile's first row until the tiles start
  if (tid < kMgCols) {
    float q2 = 0.f;
    for (int j = 0; j < r; ++j) {
      const float a = bf16_val(at[tid * AP + j]);
      q2 = __builtin_fmaf(a, a, q2);
    }
    colnorm[tid] = __fsqrt_rn(q2);
  }
  __syncthreads();

  const int64_t tiles = (g.N + kMgRows - 1) / kMgRows;
  const int64_t per_chunk = (tiles + g.row_chunks - 1) / g.row_chunks;
  const int64_t t_begin = chunk * per_chunk, t_end = min(tiles, t_begin + per_chunk);
  const int64_t kb = g.K / kBlock;
  float* urow = ut + (16 * wave) * kMgPitch;   // this wave's 16 rows of the product tile
  uint16_t* stg = reinterpret_cast<uint16_t*>(urow);   // its staging rows (after the products)
  uint32_t* list = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(urow) + kMgListOff);
  uint16_t* wb = brow[wave];

  // Lane l takes row l / 4 of the wave's 16 and columns 32 q .. +31, q = l % 4; in a last half
  // strip the lanes past it redo their neighbour's columns, and a wave whose rows lie past N (rows
  // come in 16s) redoes the last 16 rows, so that every load and store is unconditional (they
  // write identical bytes).
  const int rl = lane >> 2, q = lane & 3;
  const int cq = 32 * q < cols ? q : q - 2;
  const int64_t col = k0 + 32 * cq;
  float amax = 0.f;   // largest column norm among the lane's columns
#pragma unroll
  for (int c = 0; c < 32; ++c) amax = fmaxf(amax, colnorm[32 * cq + c]);
  __syncthreads();   // every lane has its maximum before wave 0 writes its product rows
  auto first_row = [&](int64_t t) { return min(t * kMgRows + 16 * wave, g.N - 16); };
  // per-lane parts of the addresses (the row part, first_row(t) times the row pitch, is uniform)
  const int64_t lane_p = (int64_t)rl * (g.K / 2) + col / 2;              // packed byte
  const int64_t lane_b = (int64_t)rl * kb + col / kBlock;                // scale block
  const int lane_bf = (lane & 15) * r + 4 * (lane >> 4);                 // B fragment element
  const int c16 = min(lane & 15, cols / 8 - 1);
  const int64_t lane_o = (int64_t)(lane >> 4) * g.K + k0 + 8 * c16;      // output element
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
    const uint16_t* bsrc = g.B + n0 * r + lane_bf;
#pragma unroll
    for (int s = 0; s < NT; ++s) in.bf[s] = *reinterpret_cast<const s16x4*>(bsrc + 16 * s);
    const int64_t b = n0 * kb + lane_b;
    in.p = *reinterpret_cast<const u32x4*>(g.packed + n0 * (g.K / 2) + lane_p);
    in.cw = *reinterpret_cast<const uint32_t*>(g.scale_q + (b & ~int64_t(3)));
    in.c2 = g.scale_c2[b / kGroup];
  };

  // Exact value of the listed entries list[0 .. cnt) (one per lane per round), into the staging
  // rows. Entry: column in the strip (bits 0-6), row in the wave's 16 (bits 8-11), W~ (bits 16-31).
  auto resolve = [&](int cnt) {
    for (int i = lane; i < cnt; i += 64) {
      const uint32_t ent = list[i];
      const int c = ent & 127, row = (ent >> 8) & 15;
      const uint16_t* bj = wb + row * r;
      const uint16_t* aj = at + c * AP;
      double dot = 0.0;
#pragma unroll 2
      for (int j = 0; j < r; j += 4) {
        const s16x4 bv = *reinterpret_cast<const s16x4*>(bj + j);
        const s16x4 av = *reinterpret_cast<const s16x4*>(aj + j);
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)   // the fp32 product of two bf16 values is exact
          dot += (double)(bf16_val((uint16_t)bv[i4]) * bf16_val((uint16_t)av[i4]));
      }
      stg[row * kMgStage + c] = (uint16_t)bf16_from_f64(fma((double)g.scale, dot, (double)bf16_val(ent >> 16)));
    }
  };

  auto process = [&](int64_t t, const TileIn& in, TileIn& nx, int64_t t_next) {
    const int64_t n0 = first_row(t);
    // ---- B A for rows n0 .. n0 + 15, all 128 columns; the B rows to LDS for the exact path
    f32x4 acc[kMgCols / 16];
#pragma unroll
    for (int ct = 0; ct < kMgCols / 16; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    float b2 = 0.f;   // sum of squares of this lane's j values of row lane % 16
#pragma unroll
    for (int s = 0; s < NT; ++s) {
      const int jj = 16 * s + 4 * (lane >> 4);
      *reinterpret_cast<s16x4*>(wb + (lane & 15) * r + jj) = in.bf[s];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float bv = bf16_val((uint16_t)in.bf[s][i]);
        b2 = __builtin_fmaf(bv, bv, b2);
      }
#pragma unroll
      for (int ct = 0; ct < kMgCols / 16; ++ct) {
        const s16x4 af = *reinterpret_cast<const s16x4*>(at + (ct * 16 + (lane & 15)) * AP + jj);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(af, in.bf[s], acc[ct], 0, 0, 0);
      }
    }
    b2 += __shfl_xor(b2, 16);
    b2 += __shfl_xor(b2, 32);
    // acc[ct][i] = (B A)[row lane % 16][column 16 ct + 4 (lane / 16) + i]: four consecutive columns
#pragma unroll
    for (int ct = 0; ct < kMgCols / 16; ++ct)
      *reinterpret_cast<f32x4*>(urow + (lane & 15) * kMgPitch + ct * 16 + 4 * (lane >> 4)) = acc[ct];
    if (lane < 16) urow[lane * kMgPitch + kMgCols] = b2;

    // the next tile's loads go out between this tile's MFMA part and its dequantisation, so that a
    // wave waiting for room in the CU's vector-memory queue does so with half its tile still to do
    load_tile(t_next, nx);
    __builtin_amdgcn_sched_barrier(0);

    // ---- dequantise, add, test, round
    const uint32_t b = (uint32_t)(n0 * kb) + (uint32_t)lane_b;   // low bits of the block index
    const uint32_t code = in.cw >> ((b & 3u) * 8u);              // e4m3_decode reads bits 0 .. 6
    const BlockLut lut = make_lut(__fmul_rn(e4m3_decode(code), in.c2), g.codes.v);
    const float* u = urow + rl * kMgPitch + (col - k0);
    // near-tie radius 2 |s| E for this row and these columns (rounded up by tie_coef's margin)
    const float radius = fmaxf(g.tie_coef * (__fsqrt_rn(urow[rl * kMgPitch + kMgCols]) * amax), g.tie_floor);
    uint32_t ok = 0;   // one bit per value, first value highest: set when it is clear of every tie
    u32x4 o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t p = in.p[i];
      const uint32_t odd = p & 0x0F0F0F0Fu;            // elements 1,3,5,7
      const uint32_t even = (p >> 4) & 0x0F0F0F0Fu;    // elements 0,2,4,6
      uint32_t w[8];
      lut4_f32(lut, __builtin_amdgcn_perm(odd, even, 0x05010400u), w);       // elements 0..3
      lut4_f32(lut, __builtin_amdgcn_perm(odd, even, 0x07030602u), w + 4);   // elements 4..7
      const f32x4 u0 = *reinterpret_cast<const f32x4*>(u + 8 * i);
      const f32x4 u1 = *reinterpret_cast<const f32x4*>(u + 8 * i + 4);
      const float uu[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = __builtin_fmaf(g.scale, uu[e], __uint_as_float(w[e]));
        // (bits & 0xFFFF0000) | 0x8000 as one v_bitop3 (truth table 0xEA: (a & b) | c)
        const float tie = __uint_as_float(__builtin_amdgcn_bitop3_b32(__float_as_uint(x[e]), 0xFFFF0000u, 0x8000u, 0xEA));
        const float margin = radius - fabsf(x[e] - tie);   // negative: clear of the tie
        ok = __builtin_amdgcn_alignbit(ok, __float_as_uint(margin), 31);
      }
      o[i] = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7])};
    }
    // ---- the results go into this wave's staging rows (every lane has read its product values,
    // and a wave's LDS accesses complete in order) as bf16 rows of kMgStage values
    u32x4* sdst = reinterpret_cast<u32x4*>(stg + rl * kMgStage + (col - k0));
#pragma unroll
    for (int i = 0; i < 4; ++i) sdst[i] = o[i];

    // ---- values near a tie: listed with their W~ (looked up again from the packed word), then
    // recomputed exactly over the staging rows
    uint32_t flagged = ~ok;
    if (__builtin_amdgcn_ballot_w64(flagged != 0u)) {
      int cnt = 0;   // wave-uniform
      for (;;) {
        const uint64_t m = __builtin_amdgcn_ballot_w64(flagged != 0u);
        if (!m) break;
        if (cnt + 64 > kMgListCap) {   // list full (values near ties by the thousand)
          resolve(cnt);
          cnt = 0;
        }
        if (flagged) {
          const int v = __builtin_clz(flagged);   // value v of the lane sits at bit 31 - v
          flagged &= ~(0x80000000u >> v);
          // its code: byte (v % 8) / 2 of packed word v / 8, high nibble for even v
          const uint32_t pw = v < 16 ? (v < 8 ? in.p[0] : in.p[1]) : (v < 24 ? in.p[2] : in.p[3]);
          const uint32_t idx = (pw >> (((v & 7) >> 1) * 8 + ((v & 1) ? 0 : 4))) & 15u;
          uint32_t lo, hi;
          lut4_planes(lut, idx, lo, hi);
          const uint32_t wbits = ((hi & 0xFFu) << 8) | (lo & 0xFFu);
          const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          list[cnt + below] = (wbits << 16) | ((uint32_t)rl << 8) | (uint32_t)((col - k0) + v);
        }
        cnt += __builtin_popcountll(m);
      }
      resolve(cnt);
    }

    // ---- coalesced stores: store instruction i writes rows 4 i .. 4 i + 3, 16 bytes per lane and
    // the 256 bytes of a row from 16 consecutive lanes (lanes past a half strip repeat the last
    // 16 bytes of their row, identical writes)
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const u32x4*>(stg + (4 * i + (lane >> 4)) * kMgStage + 8 * c16);
    uint16_t* orow = g.out + n0 * g.K + lane_o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4* dst = reinterpret_cast<u32x4*>(orow + 4 * i * g.K);
      if (NTSTORE) __builtin_nontemporal_store(v[i], dst);
      else *dst = v[i];
    }
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
                        int book, hipStream_t stream) {
  const int64_t strips = (K + kMgCols - 1) / kMgCols;
  const int64_t tiles = (N + kMgRows - 1) / kMgRows;
  int64_t chunks = (2048 + strips - 1) / strips;   // about 2048 workgroups in all
  if (chunks > tiles) chunks = tiles;
  if (chunks < 1) chunks = 1;
  // 4 |s| (r + 1) 2^-24, rounded up by 2^-14 to cover the roundings of the bound's own terms (the
  // norms' sums of at most 128 squares, their square roots and the products)
  const float coef = (float)(4.0 * fabs((double)scale) * (r + 1) * 0x1p-24 * (1.0 + 0x1p-14));
  const float floor_ = (float)((fabs((double)scale) + 1.0) * 0x1p-90);
  MergeArgs g{packed, scale_q, scale_c2, N, K, A, B, r, scale, coef, floor_, (int)chunks, out, {}};
  if (!codes_of(book, g.codes)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(strips * chunks)), block(256);
  switch (r / 16) {
    case 1: hipLaunchKernelGGL((qlora_merge_kernel<1, true>), grid, block, 0, stream, g); break;
    case 2: hipLaunchKernelGGL((qlora_merge_kernel<2, true>), grid, block, 0, stream, g); break;
    case 3: hipLaunchKernelGGL((qlora_merge_kernel<3, true>), grid, block, 0, stream, g); break;
    case 4: hipLaunchKernelGGL((qlora_merge_kernel<4, true>), grid, block, 0, stream, g); break;
    case 5: hipLaunchKernelGGL((qlora_merge_kernel<5, true>), grid, block, 0, stream, g); break;
    case 6: hipLaunchKernelGGL((qlora_merge_kernel<6, true>), grid, block, 0, stream, g); break;
    case 7: hipLaunchKernelGGL((qlora_merge_kernel<7, true>), grid, block, 0, stream, g); break;
    default: hipLaunchKernelGGL((qlora_merge_kernel<8, true>), grid, block, 0, stream, g); break;
  }
  return hipGetLastError();
}

}  // namespace nf4
