// Skinny forward of the adapted linear for a few tokens (M <= 16): the dequant-GEMV regime.
//
// "QLoRA, explained", The forward pass and gradients / The algorithm, step by step:
// y = x W~^T + s (x A^T) B^T. With M <= 16 the weight is read once and each dequantised value is
// used M times, so the kernel is bound by HBM bandwidth on the packed weight (0.52 bytes per
// value) and, behind it, by the dequantisation work. Layout of the work:
//   * a workgroup of 16 waves owns 256 consecutive rows of W (one 16-row tile per wave) and one
//     split of the k axis; a step covers 512 columns, and the number of splits is chosen so that
//     the (row block, split) items fill the 256 CUs once;
//   * lane (row = lane % 16, g = lane / 16) loads, with its instruction i, the 16 packed bytes at
//     offset 64 i + 16 g of its row's 256-byte step (so the four lanes of a row read 64
//     contiguous bytes per instruction): half g % 2 of block 2 i + g / 2. It dequantises them
//     straight into MFMA operand registers; dword d of that half holds columns 128 i + 32 g + 8 d
//     of the step, and the activation operand of v_mfma_f32_16x16x32_bf16 holds the same columns
//     of x[m = lane % 16], so the MFMA contracts over a permuted but consistent k order;
//   * the activations of a step (16 tokens x 512 columns) are shared by all waves: they are loaded
//     one step ahead and stored into LDS (chunk c of token t at slot c ^ t, which keeps the 16
//     token lanes of a fragment read in distinct banks; tokens past M and columns past K are
//     zeros), and one workgroup barrier per step hands them over;
//   * the packed codes, the row's eight scale codes of the step (one 16-byte load) and the
//     second-level constants of the next step are in flight in registers while a step is
//     dequantised (raw loaded words only, so issuing the loads never waits for them);
//   * dequantisation reads both codes of a packed byte from an LDS pair table (256 entries of two
//     fp32 codes, replicated 32 times so the 32 lanes of a half-wave read distinct banks): one
//     v_perm forms the address (byte * 256 + copy * 8), then two fp32 products with the block
//     scale and one bf16 pair conversion, giving bit for bit bf16(fl32(q[idx] * c1')). Four waves
//     per SIMD keep enough of these lookups in flight;
//   * u = x A^T is shared out evenly: every item forms the partial sums of u over its own slice of
//     the contraction (its split's columns cut into one run per row block), each (token, row of A)
//     pair summed by one thread in column order while the item's first weight loads are in flight.
//     (With the rows of A riding along in the items of the first row blocks instead, those items
//     read twice the bytes of the others and finished 4-8 us after them);
//   * every wave writes the fp32 partial sums of its own rows; skinny_epilogue_kernel sums the
//     split partials in split order, forms u from its partials, adds s * u B^T in fp32 and rounds
//     y to bf16.
#include "common.h"
#include "launch.h"

namespace nf4 {

constexpr int kStep = 512;                       // k columns per step
constexpr int kSkWaves = 16;                     // waves per workgroup
constexpr int kSkRows = kSkWaves * 16;           // rows of W per workgroup
constexpr int kSkSlots = 256;                    // workgroups that occupy the MI355X once

struct SkinnyArgs {
  const uint8_t* packed;
  const uint8_t* scale_q;
  const float* scale_c2;
  int64_t N, K;
  const uint16_t* x;   // [M x K] bf16
  int64_t M;
  const uint16_t* A;   // [r x K] bf16
  int r;
  SkinnyPlan p;
  float* part;         // [w_splits][M][N]
  float* upart;        // [u parts][M][r]
  const float* absmax; // fp32 block scales instead of scale_q / scale_c2
  Codes codes;         // the values the 4-bit indices select
};

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

// One step of one lane's packed weight (raw loaded values only): the bytes of instruction i are
// half g % 2 of block 2 i + g / 2.
struct SkinnyW {
  u32x4 p[4];
};
// One step of one lane's small operands, single-buffered: each is reloaded for the next step as
// soon as it has been consumed.
struct SkinnyS {
  u32x4 cw;        // 16 bytes from the aligned word holding the step's first scale code
  u32x2 c2;        // second-level constants of the step's first group and the next one
  u32x4 f0, f1;    // fp32 block scales (F32S): the step's eight blocks of the row
};

// This item's partial sums of u = x A^T: the 8-column chunks [ch0, ch1) of the contraction, for
// every token m < M and row j < r (pair p = m r + j). With P = M r pairs below 1024, the chunks are
// cut into S = min(1024 / P, ch1 - ch0) runs, thread t sums run t / P of pair t % P in column order
// into stage[t] (LDS), and after the workgroup barrier u_share_finish adds the S runs of a pair in
// run order; with more pairs, each thread sums whole pairs (t, t + 1024, ...) straight into dst.
// Either way each partial has one fixed order. The loads go out right after the item's first
// weight loads, one chunk per thread at the sizes that matter, so they add no round trip of their own.
__device__ __forceinline__ void u_share(const SkinnyArgs& g, int64_t ch0, int64_t ch1, int tid,
                                        float* __restrict__ stage, float* __restrict__ dst) {
  const int pairs = (int)g.M * g.r;
  auto sum_run = [&](int p, int64_t c0, int64_t c1) {
    const int m = p / g.r, j = p % g.r;
    const uint16_t* xr = g.x + (int64_t)m * g.K;
    const uint16_t* ar = g.A + (int64_t)j * g.K;
    float sum = 0.f;
#pragma unroll 4
    for (int64_t ch = c0; ch < c1; ++ch) {
      const u32x4 xv = *reinterpret_cast<const u32x4*>(xr + 8 * ch);
      const u32x4 av = *reinterpret_cast<const u32x4*>(ar + 8 * ch);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sum = __builtin_fmaf(__uint_as_float(xv[q] << 16), __uint_as_float(av[q] << 16), sum);
        sum = __builtin_fmaf(__uint_as_float(xv[q] & 0xFFFF0000u), __uint_as_float(av[q] & 0xFFFF0000u), sum);
      }
    }
    return sum;
  };
  if (pairs >= kSkWaves * 64) {
    for (int p = tid; p < pairs; p += kSkWaves * 64) dst[p] = sum_run(p, ch0, ch1);
    return;
  }
  const int64_t n = ch1 - ch0;
  const int runs = (int)max((int64_t)1, min((int64_t)(kSkWaves * 64 / pairs), n));
  const int run = tid / pairs;
  if (run < runs) stage[tid] = sum_run(tid % pairs, ch0 + n * run / runs, ch0 + n * (run + 1) / runs);
}

// After the barrier that follows u_share: the runs of each pair added in run order.
__device__ __forceinline__ void u_share_finish(const SkinnyArgs& g, int64_t ch0, int64_t ch1, int tid,
                                               const float* __restrict__ stage, float* __restrict__ dst) {
  const int pairs = (int)g.M * g.r;
  if (pairs >= kSkWaves * 64 || tid >= pairs) return;
  const int runs = (int)max((int64_t)1, min((int64_t)(kSkWaves * 64 / pairs), ch1 - ch0));
  float sum = 0.f;
  for (int run = 0; run < runs; ++run) sum += stage[run * pairs + tid];
  dst[tid] = sum;
}

// The chunk range of item (rb, split) for u_share: the split's columns [step s_begin, step s_end)
// (clipped at K) in 8-column chunks, cut into w_blocks runs of near-equal length.
__device__ __forceinline__ void u_chunks(const SkinnyArgs& g, int64_t step, int s_begin, int s_end, int rb,
                                         int64_t& ch0, int64_t& ch1) {
  const int64_t lo = (int64_t)s_begin * step / 8, hi = min((int64_t)s_end * step, g.K) / 8;
  const int64_t n = hi > lo ? hi - lo : 0;
  ch0 = lo + n * rb / g.p.w_blocks;
  ch1 = lo + n * (rb + 1) / g.p.w_blocks;
}

template <bool F32S>
__global__ __launch_bounds__(kSkWaves * 64) void skinny_fwd_kernel(const SkinnyArgs g) {
  __shared__ __attribute__((aligned(16))) f32x2 tab[256 * 32];
  // activation stages: 16 tokens x 64 chunks of 8 bf16
  __shared__ __attribute__((aligned(16))) u32x4 xs[2][16 * 64];
  __shared__ float ustage[kSkWaves * 64];   // runs of the u partial sums
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4;
  const int m = lane & 15;
  const uint32_t laneoff = (uint32_t)(lane & 31) * 8u;
  const int64_t nsteps = (g.K + kStep - 1) / kStep;

  // pair table: thread t fills copies 8 (t & 3) .. +7 of byte value t / 4
  {
    const int byte = tid >> 2;
    const float hi = g.codes.v[byte >> 4];
    const float lo = g.codes.v[byte & 15];
    const u32x4 v = u32x4{__float_as_uint(hi), __float_as_uint(lo), __float_as_uint(hi), __float_as_uint(lo)};
    u32x4* dst = reinterpret_cast<u32x4*>(&tab[byte * 32 + (tid & 3) * 8]);
#pragma unroll
    for (int c = 0; c < 4; ++c) dst[c] = v;
  }

  const int rb = (int)blockIdx.x % g.p.w_blocks, split = (int)blockIdx.x / g.p.w_blocks;
  const int s_begin = split * g.p.w_sub;
  const int s_end = (int)min(nsteps, (int64_t)s_begin + g.p.w_sub);
  const int64_t row = (int64_t)rb * kSkRows + wave * 16 + m;   // this lane's row of W
  const int64_t rowc = min(row, g.N - 1);
  const int64_t nblocks = g.N * (g.K / kBlock);
  const __amdgpu_buffer_rsrc_t rs_q = F32S
      ? __builtin_amdgcn_make_buffer_rsrc((void*)g.absmax, (short)0, (int)(nblocks * 4), kRsrcFlags)
      : __builtin_amdgcn_make_buffer_rsrc((void*)g.scale_q, (short)0, (int)((nblocks + 3) & ~int64_t(3)), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rs_c2 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.scale_c2, (short)0, (int)(((nblocks + kGroup - 1) / kGroup) * 4), kRsrcFlags);
  // per-lane bases, so that the step loop works with 32-bit offsets (the block count of W is
  // below 2^31, so block indices fit)
  const int kb = (int)(g.K / kBlock);                         // blocks per row
  const uint32_t rowb = (uint32_t)(rowc * kb);                // first block of this lane's row
  const uint8_t* prow = g.packed + (int64_t)rowb * 32 + 16 * (grp & 1);
  // block of instruction i of this lane in step s, within the row (clamped: blocks past K re-read
  // the row's last block, whose activations are zeros)
  auto blk_of = [&](int s, int i) { return min(s * 8 + 2 * i + (grp >> 1), kb - 1); };

  auto load_w = [&](int s, SkinnyW& st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4* src = reinterpret_cast<const u32x4*>(prow + (uint32_t)blk_of(s, i) * 32u);
      st.p[i] = __builtin_nontemporal_load(src);
    }
  };
  auto load_scales = [&](int s, SkinnyS& ss) {
    const uint32_t b0 = rowb + (uint32_t)min(s * 8, kb - 1);
    if constexpr (F32S) {
      // the step's eight blocks (past the row's end these are other rows' scales, or zeros past
      // the array; process() replaces them with zero)
      ss.f0 = __builtin_amdgcn_raw_buffer_load_b128(rs_q, b0 * 4u, 0, 0);
      ss.f1 = __builtin_amdgcn_raw_buffer_load_b128(rs_q, b0 * 4u + 16u, 0, 0);
    } else {
      ss.cw = __builtin_amdgcn_raw_buffer_load_b128(rs_q, b0 & ~3u, 0, 0);
      ss.c2 = __builtin_amdgcn_raw_buffer_load_b64(rs_c2, (b0 >> 8) * 4u, 0, 0);
    }
  };

  // activation copy: thread t moves token t / 64, slot t % 64 (source chunk slot ^ token)
  const int xt = tid >> 6, xslot = tid & 63, xchunk = xslot ^ xt;
  const uint16_t* xp = g.x + (int64_t)min(xt, (int)g.M - 1) * g.K;
  auto load_x = [&](int s) {
    const uint32_t col = (uint32_t)min((int64_t)s * kStep + 8 * xchunk, g.K - 8);
    return *reinterpret_cast<const u32x4*>(xp + col);
  };
  auto store_x = [&](int s, u32x4* stage, u32x4 v) {
    const bool live = xt < g.M && (int64_t)s * kStep + 8 * xchunk < g.K;
    stage[xt * 64 + xslot] = live ? v : u32x4{0u, 0u, 0u, 0u};
  };

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const char* tab_bytes = reinterpret_cast<const char*>(tab);

  // process step s; with `more`, the small operands of step s + 1 are loaded as soon as those of
  // step s have been consumed, and load i of step s + 1's packed weight goes out just before
  // quarter i of step s is dequantised: a wave whose load has to wait for room in the CU's
  // vector-memory queue then stalls between quarters while the other waves of its SIMD compute,
  // instead of stalling before any of its arithmetic (16 waves issuing 4 loads each at the start
  // of a step made the last waves wait about as long as the step's arithmetic)
  auto process = [&](int s, const SkinnyW& st, SkinnyW& nx, SkinnyS& ss, const u32x4* xsv, bool more) {
    const uint32_t b0 = rowb + (uint32_t)min(s * 8, kb - 1);
    const uint32_t base = b0 & 3u;   // byte of the step's first code in the 16 loaded bytes
    float c1p[4];
    if constexpr (F32S) {
      // block 2 i + grp / 2 of the step's eight
      const bool odd = (grp >> 1) != 0;
      c1p[0] = __uint_as_float(odd ? ss.f0[1] : ss.f0[0]);
      c1p[1] = __uint_as_float(odd ? ss.f0[3] : ss.f0[2]);
      c1p[2] = __uint_as_float(odd ? ss.f1[1] : ss.f1[0]);
      c1p[3] = __uint_as_float(odd ? ss.f1[3] : ss.f1[2]);
      if (s * 8 + 8 > kb) {   // the step runs past the row's end (wave-uniform)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (s * 8 + 2 * i + (grp >> 1) >= kb) c1p[i] = 0.f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t b = rowb + (uint32_t)blk_of(s, i);
        const uint32_t byte = base + (b - b0);   // < 16
        const uint32_t word = byte < 4 ? ss.cw[0] : byte < 8 ? ss.cw[1] : byte < 12 ? ss.cw[2] : ss.cw[3];
        const uint32_t code = word >> ((byte & 3u) * 8u);
        const float c2 = (b >> 8) == (b0 >> 8) ? __uint_as_float(ss.c2[0]) : __uint_as_float(ss.c2[1]);
        c1p[i] = __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)code, 0), c2);
      }
    }
    if (more) load_scales(s + 1, ss);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (more) nx.p[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(prow + (uint32_t)blk_of(s + 1, i) * 32u));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // activation fragment (i, d): chunk 16 i + 4 g + d of token m
        const bf16x8 bx = __builtin_bit_cast(bf16x8, xsv[m * 64 + ((16 * i + 4 * grp + d) ^ m)]);
        const uint32_t word = st.p[i][d];
        uint32_t a[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          // byte bb of the word holds values 8 d + 2 bb (high nibble) and + 1 of the half block
          const uint32_t off = __builtin_amdgcn_perm(word, laneoff, 0x0C0C0000u | ((4u + bb) << 8));
          const f32x2 qv = *reinterpret_cast<const f32x2*>(tab_bytes + off);
          a[bb] = pack_bf16x2(__fmul_rn(qv[0], c1p[i]), __fmul_rn(qv[1], c1p[i]));
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, (u32x4{a[0], a[1], a[2], a[3]})),
                                                      bx, acc, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Phase of step s (parity p = (s - s_begin) % 2): the activations and packed weight of s + 1 are
  // loaded (into registers; the weight a quarter at a time during the arithmetic), s is dequantised
  // and multiplied from w[p] and activation stage p, the
  // activations of s + 1 are stored into stage 1 - p (nobody reads it since the previous barrier),
  // and the barrier hands them over. Every load issued is consumed: the steady-state loop runs
  // while both of its phases have a successor, and the last one or two phases are peeled (a load
  // whose value is never used would make the compiler wait for it before reusing its registers).
  SkinnyW w[2];
  SkinnyS ss;
  int64_t uch0, uch1;
  {
    const u32x4 x0 = load_x(s_begin);
    load_w(s_begin, w[0]);
    load_scales(s_begin, ss);
    u_chunks(g, kStep, s_begin, s_end, rb, uch0, uch1);
    u_share(g, uch0, uch1, tid, ustage, g.upart + (int64_t)blockIdx.x * g.M * g.r);
    store_x(s_begin, xs[0], x0);
  }
  __syncthreads();   // the pair table, the first activation stage and the u runs are in place
  u_share_finish(g, uch0, uch1, tid, ustage, g.upart + (int64_t)blockIdx.x * g.M * g.r);
  auto phase = [&](int sp, int p, bool more) {
    u32x4 xn = u32x4{0u, 0u, 0u, 0u};
    if (more) {
      xn = load_x(sp + 1);
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the arithmetic
    process(sp, w[p], w[1 - p], ss, xs[p], more);
    if (more) store_x(sp + 1, xs[1 - p], xn);
    lds_barrier();
  };
  int sp = s_begin;
  for (; sp + 2 < s_end; sp += 2) {
    phase(sp, 0, true);
    phase(sp + 1, 1, true);
  }
  if (sp + 1 < s_end) {
    phase(sp, 0, true);
    phase(sp + 1, 1, false);
  } else {
    phase(sp, 0, false);
  }

  // acc[i]: row (tile row 4 grp + i), token m
  if (m < g.M) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r_out = (int64_t)rb * kSkRows + wave * 16 + 4 * grp + i;
      if (r_out < g.N) g.part[((int64_t)split * g.M + m) * g.N + r_out] = acc[i];
    }
  }
}

// ------------------------------------------------------------------------------------------
// M <= 4 tokens: four rows x four column chunks per MFMA.
//
// How a wave's loads map onto HBM sets the read rate of this regime: one load instruction that
// touches 16 rows (64 bytes each, the lane order of an MFMA operand) reads the weight at about
// 5.1 TB/s, one that touches 4 rows with two whole 128-byte lines each at about 6.3 TB/s. With at
// most four tokens the MFMA's 16 x 16 output can afford the second: its rows i = (rho, c) are 4
// weight rows x 4 column chunks and its columns j = (t, c') 4 tokens x the same 4 chunks, the
// chunks of an operand lane being chosen so that A row (rho, c) and B column (t, c') contract over
// the same columns exactly when c == c'. The diagonal entries c == c' are partial dot products of
// row rho with token t; the other 12 of every 16 are discarded, which costs nothing as long as
// M <= 4 (the 16-row layout wastes 16 - M of its 16 token columns just the same). After the last
// step, every lane keeps its diagonal entry and a quad of lanes sums the four chunks.
//   * a workgroup of 16 waves owns 64 rows (4 per wave) and one split of the k axis; a step is
//     2048 columns (1 KB of codes per row);
//   * lane (kg = lane / 16, rho = lane % 16 / 4, c = lane % 4), h = kg / 2: in window q = 0..3
//     of a step it loads the 16 bytes at 128 (q + 4 h) + 64 (kg % 2) + 16 c of row rho, so one
//     load instruction covers 4 rows x two whole 128-byte lines; dword d of them holds columns
//     256 (q + 4 h) + 128 (kg % 2) + 32 c + 8 d .. + 7, which is also what the activation operand
//     of (q, d) holds for token t = rho and chunk c' = c;
//   * the lane's four blocks of a step (one per window) lie 4 apart in one 16-byte window of scale
//     codes (whose start is shifted per lane by a whole dword so that it covers them); blocks past
//     the row's end get a zero scale (their activation columns are zeros as well);
//   * activations (4 tokens x 2048 columns, 16 KB) go through LDS one step ahead, and every item
//     forms its share of u, as in the 16-row kernel;
//   * with fp32 block scales (no double quantisation) the lane loads its four blocks' scales
//     directly (F32S);
//   * the split partials go to the 16-row kernel's epilogue.
constexpr int kS4Step = 2048;                    // k columns per step
constexpr int kS4Rows = kSkWaves * 4;            // rows of W per workgroup

struct Skinny4W {
  u32x4 p[4];      // window q of the step
};
struct Skinny4S {
  u32x4 cw;        // 16 scale codes: the lane's block of window q is byte p + 4 q
  u32x2 c2;        // second-level constants of the step's first group and the next one
};

template <bool F32S>
__global__ __launch_bounds__(kSkWaves * 64) void skinny4_fwd_kernel(const SkinnyArgs g) {
  __shared__ __attribute__((aligned(16))) f32x2 tab[256 * 32];
  // activation stages: 4 tokens x 256 chunks of 8 bf16; chunk k of token t sits at slot k ^ t
  __shared__ __attribute__((aligned(16))) u32x4 xs[2][4 * 256];
  __shared__ float ustage[kSkWaves * 64];   // runs of the u partial sums
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 4, hh = kg >> 1, kb2 = kg & 1;
  const int rho = (lane & 15) >> 2, c = lane & 3;
  const uint32_t laneoff = (uint32_t)(lane & 31) * 8u;
  const int64_t nsteps = (g.K + kS4Step - 1) / kS4Step;

  {
    const int byte = tid >> 2;
    const float hi = g.codes.v[byte >> 4];
    const float lo = g.codes.v[byte & 15];
    const u32x4 v = u32x4{__float_as_uint(hi), __float_as_uint(lo), __float_as_uint(hi), __float_as_uint(lo)};
    u32x4* dst = reinterpret_cast<u32x4*>(&tab[byte * 32 + (tid & 3) * 8]);
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[k] = v;
  }

  const int rb = (int)blockIdx.x % g.p.w_blocks, split = (int)blockIdx.x / g.p.w_blocks;
  const int s_begin = split * g.p.w_sub;
  const int s_end = (int)min(nsteps, (int64_t)s_begin + g.p.w_sub);
  const int64_t row = (int64_t)rb * kS4Rows + wave * 4 + rho;   // the row this lane loads
  const int64_t rowc = min(row, g.N - 1);
  const int64_t nblocks = g.N * (g.K / kBlock);
  const __amdgpu_buffer_rsrc_t rs_q = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.scale_q, (short)0, (int)((nblocks + 3) & ~int64_t(3)), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rs_c2 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.scale_c2, (short)0, (int)(((nblocks + kGroup - 1) / kGroup) * 4), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rs_am = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.absmax, (short)0, (int)(nblocks * 4), kRsrcFlags);
  const int kb = (int)(g.K / kBlock);
  const uint32_t rowb = (uint32_t)(rowc * kb);
  const int blk0 = 16 * hh + 2 * kb2 + (c >> 1);              // block of window 0 within a step
  const uint8_t* prow = g.packed + (int64_t)rowb * 32 + 16 * (c & 1);
  auto blk_of = [&](int s, int q) { return min(s * 32 + blk0 + 4 * q, kb - 1); };
  // scale window: 16 bytes from the dword holding the block of window 0 minus 0..3 bytes; since
  // 32 s + 16 hh is a multiple of 4, the lane's byte p within each dword is the same every step
  const uint32_t e0 = (rowb & 3u) + (uint32_t)(2 * kb2 + (c >> 1));   // 0..6
  const uint32_t wsh = (e0 >> 2) * 4u, pbyte = e0 & 3u;
  const uint32_t gsel = pbyte | ((pbyte + 4u) << 8);                  // bytes p of two dwords

  auto load_w = [&](int s, Skinny4W& st) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      st.p[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(prow + (uint32_t)blk_of(s, q) * 32u));
  };
  auto load_scales = [&](int s, Skinny4S& ss) {
    if constexpr (F32S) {
      // the fp32 scales of the lane's four blocks (blocks past the row's end re-read its last one)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        ss.cw[q] = __builtin_amdgcn_raw_buffer_load_b32(rs_am, (rowb + (uint32_t)blk_of(s, q)) * 4u, 0, 0);
    } else {
      const uint32_t w0 = ((rowb + (uint32_t)(32 * s + 16 * hh)) & ~3u) + wsh;
      ss.cw = __builtin_amdgcn_raw_buffer_load_b128(rs_q, w0, 0, 0);
      ss.c2 = __builtin_amdgcn_raw_buffer_load_b64(rs_c2, ((rowb + (uint32_t)(32 * s)) >> 8) * 4u, 0, 0);
    }
  };

  // activation copy: thread t moves token t / 256, chunk t % 256 (slot chunk ^ token)
  const int xt = tid >> 8, xch = tid & 255;
  const uint16_t* xp = g.x + (int64_t)min(xt, (int)g.M - 1) * g.K;
  auto load_x = [&](int s) {
    const uint32_t col = (uint32_t)min((int64_t)s * kS4Step + 8 * xch, g.K - 8);
    return *reinterpret_cast<const u32x4*>(xp + col);
  };
  auto store_x = [&](int s, u32x4* stage, u32x4 v) {
    const bool live = xt < g.M && (int64_t)s * kS4Step + 8 * xch < g.K;
    stage[xt * 256 + (xch ^ xt)] = live ? v : u32x4{0u, 0u, 0u, 0u};
  };
  // activation fragment (q, d) of this lane: token rho, chunk 32 (q + 4 hh) + 16 kb2 + 4 c + d
  const int xbase = rho * 256 + 128 * hh + 16 * kb2 + 4 * c;

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const char* tab_bytes = reinterpret_cast<const char*>(tab);

  auto process = [&](int s, const Skinny4W& st, Skinny4W& nx, Skinny4S& ss, const u32x4* xsv, bool more) {
    // block scales of the four windows
    float c1p[4];
    if constexpr (F32S) {
#pragma unroll
      for (int q = 0; q < 4; ++q) c1p[q] = __uint_as_float(ss.cw[q]);
      if (32 * s + 32 > kb) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (32 * s + blk0 + 4 * q >= kb) c1p[q] = 0.f;
      }
    } else {
      const uint32_t lo = __builtin_amdgcn_perm(ss.cw[1], ss.cw[0], gsel);
      const uint32_t hi = __builtin_amdgcn_perm(ss.cw[3], ss.cw[2], gsel);
      const uint32_t codes = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      // blocks of this step before the next group boundary
      const int bnd = 256 - (int)((rowb + (uint32_t)(32 * s)) & 255u);
      const float c2a = __uint_as_float(ss.c2[0]), c2b = __uint_as_float(ss.c2[1]);
      c1p[0] = __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)codes, 0), blk0 >= bnd ? c2b : c2a);
      c1p[1] = __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)codes, 1), blk0 + 4 >= bnd ? c2b : c2a);
      c1p[2] = __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)codes, 2), blk0 + 8 >= bnd ? c2b : c2a);
      c1p[3] = __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)codes, 3), blk0 + 12 >= bnd ? c2b : c2a);
      if (32 * s + 32 > kb) {   // the step runs past the row's end (wave-uniform)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (32 * s + blk0 + 4 * q >= kb) c1p[q] = 0.f;
      }
    }
    if (more) load_scales(s + 1, ss);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (more) nx.p[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(prow + (uint32_t)blk_of(s + 1, q) * 32u));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bf16x8 bx = __builtin_bit_cast(bf16x8, xsv[xbase + 32 * q + (d ^ rho)]);
        const uint32_t word = st.p[q][d];
        uint32_t a[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const uint32_t off = __builtin_amdgcn_perm(word, laneoff, 0x0C0C0000u | ((4u + bb) << 8));
          const f32x2 qv = *reinterpret_cast<const f32x2*>(tab_bytes + off);
          a[bb] = pack_bf16x2(__fmul_rn(qv[0], c1p[q]), __fmul_rn(qv[1], c1p[q]));
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, (u32x4{a[0], a[1], a[2], a[3]})),
                                                      bx, acc, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  Skinny4W w[2];
  Skinny4S ss;
  int64_t uch0, uch1;
  {
    const u32x4 x0 = load_x(s_begin);
    load_w(s_begin, w[0]);
    load_scales(s_begin, ss);
    u_chunks(g, kS4Step, s_begin, s_end, rb, uch0, uch1);
    u_share(g, uch0, uch1, tid, ustage, g.upart + (int64_t)blockIdx.x * g.M * g.r);
    store_x(s_begin, xs[0], x0);
  }
  __syncthreads();   // the pair table, the first activation stage and the u runs are in place
  u_share_finish(g, uch0, uch1, tid, ustage, g.upart + (int64_t)blockIdx.x * g.M * g.r);
  auto phase = [&](int sp, int p, bool more) {
    u32x4 xn = u32x4{0u, 0u, 0u, 0u};
    if (more) xn = load_x(sp + 1);
    __builtin_amdgcn_sched_barrier(0);
    process(sp, w[p], w[1 - p], ss, xs[p], more);
    if (more) store_x(sp + 1, xs[1 - p], xn);
    lds_barrier();
  };
  int sp = s_begin;
  for (; sp + 2 < s_end; sp += 2) {
    phase(sp, 0, true);
    phase(sp + 1, 1, true);
  }
  if (sp + 1 < s_end) {
    phase(sp, 0, true);
    phase(sp + 1, 1, false);
  } else {
    phase(sp, 0, false);
  }

  // lane keeps D[(kg, c)][(rho, c)]: row 4 wave + kg, token rho, chunk c; a quad sums the chunks
  auto diag_sum = [&](const f32x4& v) {
    float d = c == 0 ? v[0] : c == 1 ? v[1] : c == 2 ? v[2] : v[3];
    d += dpp_f<0xB1>(d);   // quad_perm [1,0,3,2]
    d += dpp_f<0x4E>(d);   // quad_perm [2,3,0,1]
    return d;
  };
  const float yv = diag_sum(acc);
  if (c == 0 && rho < g.M) {
    const int64_t r_out = (int64_t)rb * kS4Rows + wave * 4 + kg;
    if (r_out < g.N) g.part[((int64_t)split * g.M + rho) * g.N + r_out] = yv;
  }
}

// y[m][n] = bf16(sum_s part[s][m][n] + scale * sum_j u[m][j] B[n][j]),  u[m][j] = sum_p upart[p][m][j].
// Workgroup (x, y) = columns 256 x .. +255 of token y. It rebuilds u[y][:] in LDS: thread t sums
// the contiguous run t / r of the u partials for j = t % r, then thread j adds the runs in order,
// so every sum keeps one fixed order and the independent loads of a run are in flight together.
__global__ __launch_bounds__(256) void skinny_epilogue_kernel(const float* __restrict__ part, int splits,
                                                              const float* __restrict__ upart, int u_parts,
                                                              int64_t M, int64_t N, int r,
                                                              const uint16_t* __restrict__ B, float scale,
                                                              float* __restrict__ u_out,
                                                              uint16_t* __restrict__ y) {
  __shared__ float runs[256];
  __shared__ float us[128];
  const int64_t mm = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t n = (int64_t)blockIdx.x * 256 + tid;
  const bool live = n < N;
  // the split partials and the row of B do not depend on u: their loads go out first, so that
  // they travel together with the u partials' loads
  float ysum = 0.f;
  u32x4 bv[8];
  if (live) {
#pragma unroll 8
    for (int sp = 0; sp < splits; ++sp) ysum += part[((int64_t)sp * M + mm) * N + n];
    const u32x4* brow = reinterpret_cast<const u32x4*>(B + n * r);
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (c < r / 8) bv[c] = brow[c];
  }
  // nruns * r <= 256 and nruns * per_run >= u_parts: threads past nruns * r (r = 48, 80, 96, 112)
  // form a run past the last partial, which sums nothing and is never read
  const int nruns = 256 / r;
  const int per_run = (u_parts + nruns - 1) / nruns;
  {
    const int j = tid % r, run = tid / r;
    const int p0 = run * per_run, p1 = min(u_parts, p0 + per_run);
    float s = 0.f;
#pragma unroll 16
    for (int p = p0; p < p1; ++p) s += upart[((int64_t)p * M + mm) * r + j];
    runs[tid] = s;
  }
  __syncthreads();
  if (tid < r) {
    float s = 0.f;
    for (int run = 0; run < nruns; ++run) s += runs[run * r + tid];
    us[tid] = s;
    if (blockIdx.x == 0) u_out[mm * r + tid] = s;
  }
  __syncthreads();
  if (!live) return;
  float l = 0.f;
  const u32x4* brow = reinterpret_cast<const u32x4*>(B + n * r);
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    if (c < r / 8) {
      const u32x4 v = c < 8 ? bv[c] : brow[c];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        l = fmaf(us[8 * c + 2 * q], __uint_as_float(v[q] << 16), l);
        l = fmaf(us[8 * c + 2 * q + 1], __uint_as_float(v[q] & 0xFFFF0000u), l);
      }
    }
  }
  y[mm * N + n] = (uint16_t)(pack_bf16x2(ysum + scale * l, 0.f) & 0xFFFFu);
}

// Scale codes and second-level constants are addressed with 32-bit buffer offsets.
bool skinny_eligible(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= 16 && N * (K / kBlock) < (int64_t(1) << 31);
}

SkinnyPlan skinny_plan(int64_t M, int64_t N, int64_t K, int r) {
  SkinnyPlan p;
  p.narrow = M <= 4 ? 1 : 0;
  const int rows = p.narrow ? kS4Rows : kSkRows;
  const int64_t step = p.narrow ? kS4Step : kStep;
  const int64_t nsteps = (K + step - 1) / step;
  p.w_blocks = (int)((N + rows - 1) / rows);
  int64_t want = kSkSlots / p.w_blocks;
  if (want > nsteps) want = nsteps;
  if (want < 1) want = 1;
  p.w_sub = (int)((nsteps + want - 1) / want);
  p.w_splits = (int)((nsteps + p.w_sub - 1) / p.w_sub);
  return p;
}

// u partial sums: one per item
static int skinny_u_parts(const SkinnyPlan& p) { return p.w_splits * p.w_blocks; }

static size_t skinny_wpart_floats(const SkinnyPlan& p, int64_t M, int64_t N) {
  // the u partials start on a 16-byte boundary
  return ((size_t)p.w_splits * (size_t)M * (size_t)N + 3) & ~size_t(3);
}

size_t skinny_workspace_floats(int64_t M, int64_t N, int64_t K, int r) {
  const SkinnyPlan p = skinny_plan(M, N, K, r);
  return skinny_wpart_floats(p, M, N) + (size_t)skinny_u_parts(p) * (size_t)M * (size_t)r;
}

hipError_t launch_skinny_fwd(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                             const float* absmax, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                             const uint16_t* A, const uint16_t* B, int r, float scale, float* part,
                             float* u_out, uint16_t* y, int book, hipStream_t stream) {
  const SkinnyPlan p = skinny_plan(M, N, K, r);
  float* upart = part + skinny_wpart_floats(p, M, N);
  SkinnyArgs g{packed, scale_q, scale_c2, N, K, x, M, A, r, p, part, upart, absmax, {}};
  if (!codes_of(book, g.codes)) return hipErrorInvalidValue;
  const int items = p.w_blocks * p.w_splits;
  if (p.narrow && absmax)
    hipLaunchKernelGGL(skinny4_fwd_kernel<true>, dim3((unsigned)items), dim3(kSkWaves * 64), 0, stream, g);
  else if (p.narrow)
    hipLaunchKernelGGL(skinny4_fwd_kernel<false>, dim3((unsigned)items), dim3(kSkWaves * 64), 0, stream, g);
  else if (absmax)
    hipLaunchKernelGGL(skinny_fwd_kernel<true>, dim3((unsigned)items), dim3(kSkWaves * 64), 0, stream, g);
  else
    hipLaunchKernelGGL(skinny_fwd_kernel<false>, dim3((unsigned)items), dim3(kSkWaves * 64), 0, stream, g);
  hipLaunchKernelGGL(skinny_epilogue_kernel, dim3((unsigned)((N + 255) / 256), (unsigned)M), dim3(256), 0,
                     stream, part, p.w_splits, upart, skinny_u_parts(p), M, N, r, B, scale, u_out, y);
  return hipGetLastError();
}

}  // namespace nf4
