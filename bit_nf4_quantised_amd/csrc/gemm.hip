// Fused dequantise + bf16 MFMA GEMMs of the adapted linear (gfx950).
//
// "QLoRA, explained", The forward pass and gradients / The algorithm, step by step:
//   forward   y  = X W~^T + s (X A^T) B^T            (contraction over K)
//   backward  dX = dY W~  + s (dY B) A               (contraction over N; W is read again)
// W~ never exists in HBM: the packed NF4 codes of a tile are dequantised into LDS with the per-block
// bf16 lookup table and fed to bf16 MFMAs. The adapter term rides on the same
// accumulators as extra contraction steps: operands bf16(s * u) with B (forward) or bf16(s * v) with
// A (backward), where u = X A^T and v = dY B come from the LoRA kernels.
//
// Workgroup = 8 waves on a BM x 128 output tile, contraction in steps of 64:
//   * waves 0-3 (consumers) only read LDS and issue v_mfma_f32_32x32x16_bf16 (on gfx950 the
//     16x16x32 form issues at half that rate); each owns a (BM/2) x 64 sub-tile;
//   * waves 4-7 (producers) load the activation tile and the packed weight four steps ahead into
//     registers, dequantise the weight and write both into the LDS stage the consumers will use
//     next. With one consumer and one producer per SIMD, VALU dequantisation and global loads
//     overlap the MFMA stream.
// LDS holds two stages; one workgroup barrier per step separates "consumers read stage s" from
// "producers write stage s+1".
//
// The W tile in LDS is stored [row of W][column of W] (K contiguous) for both directions: the
// forward reads it row-wise with ds_read_b128, the backward reads it column-wise with
// ds_read_b64_tr_b16 (within 16 lanes, lane j receives element j%4 of the 8-byte rows addressed by
// lanes j/4, j/4+4, j/4+8 and j/4+12).
#include "common.h"
#include "launch.h"

namespace nf4 {

struct GemmArgs {
  const uint8_t* packed;
  const uint8_t* scale_q;
  const float* scale_c2;
  int64_t N, K;             // W is N x K
  const uint16_t* act;      // X [M x K] (forward) or dY [M x N] (backward), bf16
  int64_t M;
  const float* lora_act;    // u [M x r] (forward) or v [M x r] (backward), fp32
  const uint16_t* lora_w;   // B [N x r] (forward) or A [r x K] (backward), bf16
  int r;
  float scale;
  uint16_t* out;            // y [M x N] (forward) or dX [M x K] (backward), bf16
};

constexpr int kBN = 128;      // output columns per tile
constexpr int kBK = 64;       // contraction per step
constexpr int kAP = kBK + 8;  // activation tile pitch (bf16 elements)

template <bool DX>
struct WTile {
  static constexpr int rows = DX ? kBK : kBN;            // contraction rows (DX) or output rows
  // pitches keep the rows of one 16-lane LDS access in distinct banks (dX: 288-byte rows, so the
  // four rows a transpose read touches sit 32 bytes apart modulo 128)
  static constexpr int pitch = DX ? kBN + 16 : kBK + 8;
  static constexpr int segs = DX ? kBN / 32 : kBK / 32;  // 32-value segments per row
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <bool DX, int BM>
struct Smem {
  uint16_t A[2][BM][kAP];
  uint16_t W[2][WTile<DX>::rows][WTile<DX>::pitch];
};

// Producer-side staging of one contraction step in registers. Only raw loaded values are held
// here (no arithmetic on them), so issuing the loads never waits for their arrival.
template <int NA>
struct Staged {
  u32x4 act[NA];
  u32x4 wq;        // 32 packed codes
  uint32_t wcode;  // E4M3 code of their block's scale
  float wc2;       // the block's second-level constant
};

template <bool DX, int BM>
__global__ __launch_bounds__(512) void qlora_gemm_kernel(const GemmArgs g) {
  constexpr int WM = BM / 2, WN = kBN / 2;   // consumer sub-tile
  constexpr int TM = WM / 32, TN = WN / 32;  // 32 x 32 MFMA tiles per consumer
  constexpr int NA = BM * kBK / 8 / 256;     // 16-byte activation chunks per producer thread
  using WT = WTile<DX>;

  __shared__ __attribute__((aligned(16))) Smem<DX, BM> sm;

  const int tid = threadIdx.x;
  const bool producer = tid >= 256;
  const int lane = tid & 63, wave = (tid >> 6) & 3;
  const int pt = tid - 256;  // producer thread index (valid if producer)

  // Tile coordinates; workgroups are dealt round-robin over the 8 XCDs, so give each XCD a
  // contiguous run of tiles that share an activation row block.
  const int gx = gridDim.x, total = gridDim.x * gridDim.y;
  int lin = blockIdx.x + gx * blockIdx.y;
  if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
  const int64_t col0 = (int64_t)(lin % gx) * kBN;
  const int64_t m0 = (int64_t)(lin / gx) * BM;

  const int64_t Lc = DX ? g.N : g.K;       // contraction length
  const int64_t Nout = DX ? g.K : g.N;     // output columns
  const int main_steps = (int)((Lc + kBK - 1) / kBK);
  const int lora_steps = (g.r + kBK - 1) / kBK;
  const int steps = main_steps + lora_steps;

  // ---------------------------------------------------------------- producer helpers
  // Loads are never predicated: addresses are clamped into range and the data of out-of-range
  // chunks is zeroed when it is written to LDS. With straight-line loads the compiler can count
  // outstanding loads exactly and waits only for the step being written, keeping the later
  // steps in flight.
  const int w_row = pt / WT::segs, w_seg = pt % WT::segs;

  auto load_main = [&](int s, Staged<NA>& st) {
    const int64_t c0 = (int64_t)s * kBK;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int q = pt + 256 * i;
      const int64_t row = min(m0 + (q >> 3), g.M - 1);
      const int64_t col = min(c0 + (q & 7) * 8, Lc - 8);
      st.act[i] = *reinterpret_cast<const u32x4*>(g.act + row * Lc + col);
    }
    int64_t n, k;
    if (DX) { n = c0 + w_row; k = col0 + 32 * w_seg; }
    else    { n = col0 + w_row; k = c0 + 32 * w_seg; }
    n = min(n, g.N - 1);
    k = min(k, g.K - 32);
    const int64_t e = n * g.K + k;
    const int64_t b = e / kBlock;
    st.wq = *reinterpret_cast<const u32x4*>(g.packed + e / 2);
    st.wcode = g.scale_q[b];
    st.wc2 = g.scale_c2[b / kGroup];
  };

  // whole-tile bounds tests are uniform across the workgroup; per-chunk tests only on edge tiles
  const bool rows_full = m0 + BM <= g.M;
  auto store_main = [&](int s, int buf, const Staged<NA>& st) {
    const int64_t c0 = (int64_t)s * kBK;
    const bool act_full = rows_full && c0 + kBK <= Lc;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int q = pt + 256 * i;
      u32x4 v = st.act[i];
      if (!act_full) {
        const bool ok = m0 + (q >> 3) < g.M && c0 + (q & 7) * 8 < Lc;
        if (!ok) v = u32x4{0u, 0u, 0u, 0u};
      }
      *reinterpret_cast<u32x4*>(&sm.A[buf][q >> 3][(q & 7) * 8]) = v;
    }
    int64_t n, k;
    if (DX) { n = c0 + w_row; k = col0 + 32 * w_seg; }
    else    { n = col0 + w_row; k = c0 + 32 * w_seg; }
    const bool w_full = DX ? (c0 + kBK <= g.N && col0 + kBN <= g.K) : (col0 + kBN <= g.N);
    const bool wvalid = w_full || (n < g.N && k < g.K);
    u32x4* dst = reinterpret_cast<u32x4*>(&sm.W[buf][w_row][32 * w_seg]);
    const BlockLut t = make_lut(__fmul_rn(e4m3_decode(st.wcode), st.wc2));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t d[4];
      dequant8(t, st.wq[i], d);
      u32x4 v = u32x4{d[0], d[1], d[2], d[3]};
      if (!w_full && !wvalid) v = u32x4{0u, 0u, 0u, 0u};
      dst[i] = v;
    }
  };

  // adapter step: contraction over rank columns j0 .. j0+63, loaded straight into LDS
  auto store_lora = [&](int s, int buf) {
    const int j0 = (s - main_steps) * kBK;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int q = pt + 256 * i;
      const int64_t row = m0 + (q >> 3);
      const int col = j0 + (q & 7) * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (row < g.M && col < g.r) {
        const f32x4* src = reinterpret_cast<const f32x4*>(g.lora_act + row * g.r + col);
        const f32x4 a = src[0], b = src[1];
        const float sc = g.scale;
        v = u32x4{pack_bf16x2(sc * a[0], sc * a[1]), pack_bf16x2(sc * a[2], sc * a[3]),
                  pack_bf16x2(sc * b[0], sc * b[1]), pack_bf16x2(sc * b[2], sc * b[3])};
      }
      *reinterpret_cast<u32x4*>(&sm.A[buf][q >> 3][(q & 7) * 8]) = v;
    }
    u32x4* dst = reinterpret_cast<u32x4*>(&sm.W[buf][w_row][32 * w_seg]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (DX) {
        const int64_t j = j0 + w_row, k = col0 + 32 * w_seg + 8 * i;
        if (j < g.r && k < g.K) v = *reinterpret_cast<const u32x4*>(g.lora_w + j * g.K + k);
      } else {
        const int64_t n = col0 + w_row;
        const int j = j0 + 32 * w_seg + 8 * i;
        if (n < g.N && j < g.r) v = *reinterpret_cast<const u32x4*>(g.lora_w + n * g.r + j);
      }
      dst[i] = v;
    }
  };

  // ---------------------------------------------------------------- producer loop
  // The two roles run separate loops that execute the same number of workgroup barriers
  // (1 + steps), so each role's registers are live only in its own loop. Producers keep a ring of
  // four register stages (slot k holds main step t with t % 4 == k; loads past the last main step
  // re-read it, unused): at step s they dequantise step s+1 into LDS and start loading step s+5
  // into the slot just freed, so each load has about four steps to arrive.
  if (producer) {
    const int last = main_steps - 1;
    Staged<NA> r0, r1, r2, r3;
    load_main(0, r0);
    load_main(min(1, last), r1);
    load_main(min(2, last), r2);
    load_main(min(3, last), r3);
    store_main(0, 0, r0);
    load_main(min(4, last), r0);
    __syncthreads();
    auto body = [&](int s, Staged<NA>& next) {  // s + 1 < main_steps; `next` holds step s+1
      store_main(s + 1, (s + 1) & 1, next);
      load_main(min(s + 5, last), next);
      __syncthreads();
    };
    for (int s = 0; s < last; s += 4) {
      body(s, r1);
      if (s + 1 >= last) break;
      body(s + 1, r2);
      if (s + 2 >= last) break;
      body(s + 2, r3);
      if (s + 3 >= last) break;
      body(s + 3, r0);
    }
    // adapter steps, then the barrier of the final step
    for (int s = last; s < steps - 1; ++s) {
      store_lora(s + 1, (s + 1) & 1);
      __syncthreads();
    }
    __syncthreads();
    return;
  }

  // ---------------------------------------------------------------- consumer loop
  // v_mfma_f32_32x32x16_bf16 (the full-rate bf16 MFMA on gfx950): operand lane l holds row/column
  // l % 32 and contraction 8 * (l / 32) .. +7; the result lane l holds column l % 32 and rows
  // 8 * (q / 4) + 4 * (l / 32) + q % 4 for register q. The weight operand is the row side, so a lane
  // ends up with four consecutive output columns of one activation row.
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
  f32x16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  auto load_frags = [&](int buf, int kk, bf16x8* afr, bf16x8* bfr) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
      bfr[tm] = *reinterpret_cast<const bf16x8*>(
          &sm.A[buf][wm0 + tm * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      if (DX) {
        // two 16-lane transpose loads per operand: lane group g16 covers output columns
        // (g16 & 1) * 16 .. +15 and contraction rows 8 * (g16 >> 1) .. +7
        const int j = lane & 15, g16 = lane >> 4;
        const int col = wn0 + tn * 32 + (g16 & 1) * 16 + 4 * (j & 3);
        const int row = kk + (g16 >> 1) * 8 + (j >> 2);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(&sm.W[buf][row][col]));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(&sm.W[buf][row + 4][col]));
        afr[tn] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      } else {
        afr[tn] = *reinterpret_cast<const bf16x8*>(
            &sm.W[buf][wn0 + tn * 32 + (lane & 31)][kk + 8 * (lane >> 5)]);
      }
    }
  };

  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 16) {
      bf16x8 afr[TN], bfr[TM];
      load_frags(buf, kk, afr, bfr);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[tn], bfr[tm], acc[tn][tm], 0, 0, 0);
    }
  };

  __syncthreads();
  for (int s = 0; s < steps; ++s) {
    compute(s & 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int64_t m = m0 + wm0 + tm * 32 + (lane & 31);
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int64_t n = col0 + wn0 + tn * 32 + 8 * rq + 4 * (lane >> 5);
        if (m < g.M && n < Nout) {
          const f32x16& a = acc[tn][tm];
          *reinterpret_cast<u32x2*>(g.out + m * Nout + n) =
              u32x2{pack_bf16x2(a[4 * rq], a[4 * rq + 1]), pack_bf16x2(a[4 * rq + 2], a[4 * rq + 3])};
        }
      }
    }
  }
}

template <bool DX>
static hipError_t launch_gemm_t(const GemmArgs& g, hipStream_t stream) {
  const int64_t Nout = DX ? g.K : g.N;
  const int gx = (int)((Nout + kBN - 1) / kBN);
  const int64_t tiles256 = (int64_t)gx * ((g.M + 255) / 256);
  if (g.M > 128 && tiles256 >= 192) {
    const int gy = (int)((g.M + 255) / 256);
    hipLaunchKernelGGL((qlora_gemm_kernel<DX, 256>), dim3(gx, gy), dim3(512), 0, stream, g);
  } else if (g.M > 64) {
    const int gy = (int)((g.M + 127) / 128);
    hipLaunchKernelGGL((qlora_gemm_kernel<DX, 128>), dim3(gx, gy), dim3(512), 0, stream, g);
  } else {
    const int gy = (int)((g.M + 63) / 64);
    hipLaunchKernelGGL((qlora_gemm_kernel<DX, 64>), dim3(gx, gy), dim3(512), 0, stream, g);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_gemm(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                           int64_t N, int64_t K, const uint16_t* x, int64_t M, const float* u,
                           const uint16_t* B, int r, float scale, uint16_t* y, hipStream_t stream) {
  GemmArgs g{packed, scale_q, scale_c2, N, K, x, M, u, B, r, scale, y};
  return launch_gemm_t<false>(g, stream);
}

hipError_t launch_dx_gemm(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                          int64_t N, int64_t K, const uint16_t* dy, int64_t M, const float* v,
                          const uint16_t* A, int r, float scale, uint16_t* dx, hipStream_t stream) {
  GemmArgs g{packed, scale_q, scale_c2, N, K, dy, M, v, A, r, scale, dx};
  return launch_gemm_t<true>(g, stream);
}

}  // namespace nf4
