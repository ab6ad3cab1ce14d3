// Skinny forward of the adapted linear for a few tokens (M <= 16): the dequant-GEMV regime.
//
// "QLoRA, explained", The forward pass and gradients / The algorithm, step by step:
// y = x W~^T + s (x A^T) B^T. With M <= 16 the weight is read once and each dequantised value is
// used M times, so the kernel is bound by HBM bandwidth on the packed weight (0.52 bytes per
// value) and, behind it, by the dequantisation work. Layout of the work:
//   * a workgroup of 16 waves owns 512 consecutive rows of W (32 per wave, two 16-row tiles) and
//     one split of the k axis; the splits are whole 256-column sub-chunks, and their number is
//     chosen so that the (row block, split) items fill the 256 CUs once;
//   * lane (row = lane % 16, grp = lane / 16) dequantises the 64-value block at column
//     kb + 64 * grp of its row straight into MFMA operand registers; the activation operand of
//     v_mfma_f32_16x16x32_bf16 holds x[m = lane % 16][kb + 64 * grp ...], so the MFMA contracts
//     over a permuted but consistent k order;
//   * the activations of a sub-chunk (16 tokens x 256 columns) are shared by all waves: they are
//     loaded one sub-chunk ahead and stored into LDS (chunk c of token t at slot c ^ t, which keeps
//     the 16 token lanes of a fragment read in distinct banks; tokens past M and columns past K are
//     zeros), and one workgroup barrier per sub-chunk hands them over;
//   * the packed codes of the next sub-chunk are in flight in registers while a sub-chunk is
//     dequantised (raw loaded words only, so issuing the loads never waits for them);
//   * dequantisation reads both codes of a packed byte from an LDS pair table (256 entries of two
//     fp32 codes, replicated 32 times so the 32 lanes of a half-wave read distinct banks): one
//     v_perm forms the address (byte * 256 + copy * 8), then two fp32 products with the block
//     scale and one bf16 pair conversion, giving bit for bit bf16(fl32(q[idx] * c1')). Four waves
//     per SIMD keep enough of these lookups in flight;
//   * every wave writes the fp32 partial sums of its own rows; the r rows of A (bf16, no
//     dequantisation) are handled by separate small items, dispatched first, that write partial
//     sums of u = x A^T;
//   * skinny_epilogue_kernel sums the split partials in split order, forms u from its partials,
//     adds s * u B^T in fp32 and rounds y to bf16.
#include "common.h"
#include "launch.h"

namespace nf4 {

constexpr int kSub = 256;                        // k columns per sub-chunk
constexpr int kSkWaves = 16;                     // waves per workgroup
constexpr int kSkTN = 2;                         // 16-row tiles per wave
constexpr int kSkRows = kSkWaves * kSkTN * 16;   // rows of W per workgroup
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
  float* upart;        // [a_items * 16][M][r]
};

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

// One sub-chunk of one lane's weight operands (raw loaded values only).
struct SkinnyW {
  u32x4 p[kSkTN][2];   // [tile][half of the lane's 64-value block]
  uint32_t cw[kSkTN];  // aligned words holding the E4M3 codes of the block scales
  float c2[kSkTN];     // second-level constants
};

__constant__ uint32_t kSkinnyCodes[16] = {NF4_CODE_BITS};

__global__ __launch_bounds__(kSkWaves * 64) void skinny_fwd_kernel(const SkinnyArgs g) {
  __shared__ __attribute__((aligned(16))) f32x2 tab[256 * 32];
  // activation stages: 16 tokens x 32 chunks of 8 bf16
  __shared__ __attribute__((aligned(16))) u32x4 xs[2][16 * 32];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4;
  const int m = lane & 15;
  const uint32_t laneoff = (uint32_t)(lane & 31) * 8u;
  const int64_t nsub = (g.K + kSub - 1) / kSub;

  // pair table: thread t fills copies 8 (t & 3) .. +7 of byte value t / 4
  {
    const int byte = tid >> 2;
    const float hi = __uint_as_float(kSkinnyCodes[byte >> 4]);
    const float lo = __uint_as_float(kSkinnyCodes[byte & 15]);
    const u32x4 v = u32x4{__float_as_uint(hi), __float_as_uint(lo), __float_as_uint(hi), __float_as_uint(lo)};
    u32x4* dst = reinterpret_cast<u32x4*>(&tab[byte * 32 + (tid & 3) * 8]);
#pragma unroll
    for (int c = 0; c < 4; ++c) dst[c] = v;
  }

  const int a_items = g.p.a_items;
  if ((int)blockIdx.x < a_items) {
    // ---------------------------------------------------------------- adapter rows: u partials
    // wave w takes sub-chunk 16 * item + w of every 16-row tile of A; activations from global
    const int64_t sub = (int64_t)blockIdx.x * kSkWaves + wave;
    const int64_t kk0 = sub * kSub + 64 * grp;
    const bool live = sub < nsub;
    const int64_t kk = min(kk0, g.K - 64);
    bf16x8 b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = bf16x8{};
    if (live && m < g.M && kk0 < g.K) {
      const bf16x8* src = reinterpret_cast<const bf16x8*>(g.x + (int64_t)m * g.K + kk0);
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = src[j];
    }
    float* dst = g.upart + ((int64_t)blockIdx.x * kSkWaves + wave) * g.M * g.r;
    for (int t0 = 0; t0 < g.r; t0 += 16) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      if (live) {
        const u32x4* src = reinterpret_cast<const u32x4*>(g.A + (int64_t)(t0 + (lane & 15)) * g.K + kk);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, src[i]), b[i], acc, 0, 0, 0);
      }
      // acc[i]: row t0 + 4 grp + i of A, token m
      if (m < g.M) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(int64_t)m * g.r + t0 + 4 * grp + i] = acc[i];
      }
    }
    return;
  }

  // ------------------------------------------------------------------ weight rows
  const int it = (int)blockIdx.x - a_items;
  const int rb = it % g.p.w_blocks, split = it / g.p.w_blocks;
  const int64_t s_begin = (int64_t)split * g.p.w_sub;
  const int64_t s_end = min(nsub, s_begin + g.p.w_sub);
  const int64_t row0 = (int64_t)rb * kSkRows + wave * (kSkTN * 16);
  const uint32_t kb = (uint32_t)(g.K / kBlock);
  int64_t rowc[kSkTN];
#pragma unroll
  for (int tn = 0; tn < kSkTN; ++tn) rowc[tn] = min(row0 + tn * 16 + (lane & 15), g.N - 1);

  // activation copy: wave w moves tokens 2 (w % 8), +1 of a sub-chunk (lane i: token
  // 2 (w % 8) + i / 32, slot i % 32 of the token's row, source chunk slot ^ token); tokens past M
  // and columns past K are zeros. Waves w and w + 8 store the same values, so that every wave runs
  // the same code. The copy goes through registers: loaded at the start of the phase before the
  // sub-chunk is used, stored into LDS at its end.
  // The load itself is unconditional (clamped into range) and the zeros are selected at the store:
  // a load that some lanes skip would make the compiler wait for every load in flight.
  const int xt = 2 * (wave & 7) + (lane >> 5), xslot = lane & 31, xchunk = xslot ^ (xt & 15);
  const int64_t xrow = (int64_t)min(xt, (int)g.M - 1) * g.K;
  auto load_x = [&](int64_t sub) {
    const int64_t col = min(sub * kSub + 8 * xchunk, g.K - 8);
    return *reinterpret_cast<const u32x4*>(g.x + xrow + col);
  };
  auto store_x = [&](int64_t sub, u32x4* stage, u32x4 v) {
    const bool live = xt < g.M && sub * kSub + 8 * xchunk < g.K;
    stage[xt * 32 + xslot] = live ? v : u32x4{0u, 0u, 0u, 0u};
  };

  // weight loads of one sub-chunk; blocks past K re-read the last block of the row (their
  // activations are zeros)
  auto load_w = [&](int64_t sub, SkinnyW& st) {
    const int64_t kk = min(sub * kSub + 64 * grp, g.K - 64);
#pragma unroll
    for (int tn = 0; tn < kSkTN; ++tn) {
      const int64_t e = rowc[tn] * g.K + kk;
      const u32x4* src = reinterpret_cast<const u32x4*>(g.packed + e / 2);
      st.p[tn][0] = __builtin_nontemporal_load(src);
      st.p[tn][1] = __builtin_nontemporal_load(src + 1);
      const int64_t b = e / kBlock;
      // the aligned word holding the code (it never crosses a page, and its other bytes are
      // ignored), so no byte extraction has to wait for the load
      st.cw[tn] = *reinterpret_cast<const uint32_t*>(g.scale_q + (b & ~int64_t(3)));
      st.c2[tn] = g.scale_c2[b / kGroup];
    }
  };

  f32x4 acc[kSkTN];
#pragma unroll
  for (int i = 0; i < kSkTN; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const char* tab_bytes = reinterpret_cast<const char*>(tab);

  auto process = [&](int64_t sub, const SkinnyW& st, const u32x4* xsv) {
    const int64_t kk = min(sub * kSub + 64 * grp, g.K - 64);
    float c1p[kSkTN];
#pragma unroll
    for (int tn = 0; tn < kSkTN; ++tn) {
      const uint32_t b = (uint32_t)rowc[tn] * kb + (uint32_t)(kk / kBlock);
      c1p[tn] = __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)(st.cw[tn] >> ((b & 3u) * 8u)), 0), st.c2[tn]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // activation fragment i: chunk 8 grp + i of token m
      const bf16x8 bx = __builtin_bit_cast(bf16x8, xsv[m * 32 + ((8 * grp + i) ^ m)]);
#pragma unroll
      for (int tn = 0; tn < kSkTN; ++tn) {
        const uint32_t word = st.p[tn][i >> 2][i & 3];
        uint32_t a[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          // byte bb of the word holds values 8 i + 2 bb (high nibble) and + 1
          const uint32_t off = __builtin_amdgcn_perm(word, laneoff, 0x0C0C0000u | ((4u + bb) << 8));
          const f32x2 qv = *reinterpret_cast<const f32x2*>(tab_bytes + off);
          a[bb] = pack_bf16x2(__fmul_rn(qv[0], c1p[tn]), __fmul_rn(qv[1], c1p[tn]));
        }
        acc[tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, (u32x4{a[0], a[1], a[2], a[3]})),
                                                          bx, acc[tn], 0, 0, 0);
      }
    }
  };

  // Phase of sub-chunk s (parity p = (s - s_begin) % 2): the activations and weights of s + 1 are
  // loaded (into registers), s is dequantised and multiplied from w[p] and activation stage p, the
  // activations of s + 1 are stored into stage 1 - p (nobody reads it since the previous barrier),
  // and the barrier hands them over. Every load issued is consumed: the steady-state loop runs
  // while both of its phases have a successor, and the last one or two phases are peeled.
  SkinnyW w[2];
  {
    const u32x4 x0 = load_x(s_begin);
    load_w(s_begin, w[0]);
    store_x(s_begin, xs[0], x0);
  }
  __syncthreads();   // the pair table and the first activation stage are in place
  auto phase = [&](int64_t sp, int p, bool more) {
    u32x4 xn = u32x4{0u, 0u, 0u, 0u};
    if (more) {
      xn = load_x(sp + 1);
      load_w(sp + 1, w[1 - p]);
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the arithmetic
    process(sp, w[p], xs[p]);
    if (more) store_x(sp + 1, xs[1 - p], xn);
    lds_barrier();
  };
  int64_t sp = s_begin;
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

  // acc[tn][i]: row row0 + 16 tn + 4 grp + i, token m
  if (m < g.M) {
#pragma unroll
    for (int tn = 0; tn < kSkTN; ++tn)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = row0 + tn * 16 + 4 * grp + i;
        if (row < g.N) g.part[((int64_t)split * g.M + m) * g.N + row] = acc[tn][i];
      }
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
  const int nruns = 256 / r;                          // r divides 256 (r % 16 == 0, r <= 128)
  const int per_run = (u_parts + nruns - 1) / nruns;
  {
    const int j = tid % r, run = tid / r;
    const int p0 = run * per_run, p1 = min(u_parts, p0 + per_run);
    float s = 0.f;
#pragma unroll 8
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
  const int64_t n = (int64_t)blockIdx.x * 256 + tid;
  if (n >= N) return;
  float s = 0.f;
#pragma unroll 8
  for (int sp = 0; sp < splits; ++sp) s += part[((int64_t)sp * M + mm) * N + n];
  float l = 0.f;
  const u32x4* brow = reinterpret_cast<const u32x4*>(B + n * r);
  for (int c = 0; c < r / 8; ++c) {
    const u32x4 v = brow[c];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      l = fmaf(us[8 * c + 2 * q], __uint_as_float(v[q] << 16), l);
      l = fmaf(us[8 * c + 2 * q + 1], __uint_as_float(v[q] & 0xFFFF0000u), l);
    }
  }
  y[mm * N + n] = (uint16_t)(pack_bf16x2(s + scale * l, 0.f) & 0xFFFFu);
}

// The activation copy addresses x with 32-bit buffer offsets.
bool skinny_eligible(int64_t M, int64_t K) { return M >= 1 && M <= 16 && M * K * 2 < (int64_t(1) << 31); }

SkinnyPlan skinny_plan(int64_t N, int64_t K, int r) {
  SkinnyPlan p;
  const int64_t nsub = (K + kSub - 1) / kSub;
  p.w_blocks = (int)((N + kSkRows - 1) / kSkRows);
  int64_t want = kSkSlots / p.w_blocks;
  if (want > nsub) want = nsub;
  if (want < 1) want = 1;
  p.w_sub = (int)((nsub + want - 1) / want);
  p.w_splits = (int)((nsub + p.w_sub - 1) / p.w_sub);
  p.a_items = (int)((nsub + kSkWaves - 1) / kSkWaves);
  (void)r;
  return p;
}

static size_t skinny_wpart_floats(const SkinnyPlan& p, int64_t M, int64_t N) {
  // the u partials start on a 16-byte boundary
  return ((size_t)p.w_splits * (size_t)M * (size_t)N + 3) & ~size_t(3);
}

size_t skinny_workspace_floats(int64_t M, int64_t N, int64_t K, int r) {
  const SkinnyPlan p = skinny_plan(N, K, r);
  return skinny_wpart_floats(p, M, N) + (size_t)p.a_items * kSkWaves * (size_t)M * (size_t)r;
}

hipError_t launch_skinny_fwd(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                             int64_t N, int64_t K, const uint16_t* x, int64_t M, const uint16_t* A,
                             const uint16_t* B, int r, float scale, float* part, float* u_out,
                             uint16_t* y, hipStream_t stream) {
  const SkinnyPlan p = skinny_plan(N, K, r);
  float* upart = part + skinny_wpart_floats(p, M, N);
  SkinnyArgs g{packed, scale_q, scale_c2, N, K, x, M, A, r, p, part, upart};
  const int items = p.a_items + p.w_blocks * p.w_splits;
  hipLaunchKernelGGL(skinny_fwd_kernel, dim3((unsigned)items), dim3(kSkWaves * 64), 0, stream, g);
  hipLaunchKernelGGL(skinny_epilogue_kernel, dim3((unsigned)((N + 255) / 256), (unsigned)M), dim3(256), 0,
                     stream, part, p.w_splits, upart, p.a_items * kSkWaves, M, N, r, B, scale, u_out, y);
  return hipGetLastError();
}

}  // namespace nf4
