// Fused dequantise + bf16 MFMA GEMMs of the adapted linear (gfx950).
//
// "QLoRA, explained", The forward pass and gradients / The algorithm, step by step:
//   forward   y  = X W~^T + s (X A^T) B^T            (contraction over K)
//   backward  dX = dY W~  + s (dY B) A               (contraction over N; W is read again)
// W~ never exists in HBM: each workgroup dequantises a tile of packed NF4 codes into LDS with the
// per-block bf16 lookup table and feeds it to v_mfma_f32_16x16x32_bf16. The adapter term rides on
// the same accumulators as extra contraction steps: the operands are bf16(s * u) with B (forward)
// or bf16(s * v) with A (backward), where u = X A^T and v = dY B come from the LoRA kernels.
//
// Tile: BM activation rows x 128 output columns, contraction in steps of 64. The W tile in LDS is
// stored [row of W][column of W] (K contiguous) for both directions: the forward reads it row-wise
// with ds_read_b128, the backward reads it column-wise with ds_read_b64_tr_b16 (a 16-lane
// transpose load: lane j of a 16-lane group receives element j%4 of the 8-byte rows addressed by
// lanes j/4, j/4+4, j/4+8, j/4+12).
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

constexpr int kBN = 128;   // output columns per tile
constexpr int kBK = 64;    // contraction per step
constexpr int kAP = kBK + 8;  // activation tile pitch (bf16 elements)

template <bool DX>
struct WTile {
  static constexpr int rows = DX ? kBK : kBN;        // contraction rows (DX) or output rows
  static constexpr int pitch = DX ? kBN + 8 : kBK + 8;
  static constexpr int segs = DX ? kBN / 32 : kBK / 32;  // 32-element segments per row
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <bool DX, int BM>
__global__ __launch_bounds__(256) void qlora_gemm_kernel(const GemmArgs g) {
  constexpr int WAVES_M = BM >= 128 ? 2 : 1;
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = kBN / WAVES_N;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int NA = BM * kBK / 8 / 256;  // 16-byte activation chunks per thread per step
  using WT = WTile<DX>;

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][kAP];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][WT::rows][WT::pitch];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / WAVES_N) * WM, wn0 = (wave % WAVES_N) * WN;

  // Tile coordinates; workgroups are dealt round-robin over the 8 XCDs, so give each XCD a
  // contiguous run of tiles that share an activation row block.
  const int gx = gridDim.x, total = gridDim.x * gridDim.y;
  int lin = blockIdx.x + gx * blockIdx.y;
  if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
  const int64_t col0 = (int64_t)(lin % gx) * kBN;
  const int64_t m0 = (int64_t)(lin / gx) * BM;

  const int64_t Lc = DX ? g.N : g.K;           // contraction length
  const int64_t Nout = DX ? g.K : g.N;         // output columns
  const int64_t ld_act = Lc;
  const int steps = (int)((Lc + kBK - 1) / kBK);

  f32x4 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- per-thread roles for staging
  // activation: chunk q = tid + 256 * i covers row q / 8, columns (q % 8) * 8 .. +8
  // W: thread covers one 32-element segment of one tile row
  const int w_row = tid / WT::segs, w_seg = tid % WT::segs;

  u32x4 areg[NA];
  u32x4 wreg;
  float wscale;
  bool wvalid;

  auto load_step = [&](int s) {
    const int64_t c0 = (int64_t)s * kBK;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int q = tid + 256 * i;
      const int64_t row = m0 + (q >> 3), col = c0 + (q & 7) * 8;
      if (row < g.M && col < Lc)
        areg[i] = *reinterpret_cast<const u32x4*>(g.act + row * ld_act + col);
      else
        areg[i] = u32x4{0u, 0u, 0u, 0u};
    }
    int64_t n, k;
    if (DX) { n = c0 + w_row; k = col0 + 32 * w_seg; }
    else    { n = col0 + w_row; k = c0 + 32 * w_seg; }
    wvalid = n < g.N && k < g.K;
    if (wvalid) {
      const int64_t e = n * g.K + k;
      wreg = *reinterpret_cast<const u32x4*>(g.packed + e / 2);
      wscale = block_scale(g.scale_q, g.scale_c2, e / kBlock);
    }
  };

  auto store_step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int q = tid + 256 * i;
      *reinterpret_cast<u32x4*>(&As[buf][q >> 3][(q & 7) * 8]) = areg[i];
    }
    u32x4* dst = reinterpret_cast<u32x4*>(&Ws[buf][w_row][32 * w_seg]);
    if (wvalid) {
      const BlockLut t = make_lut(wscale);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t d[4];
        dequant8(t, wreg[i], d);
        dst[i] = u32x4{d[0], d[1], d[2], d[3]};
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = u32x4{0u, 0u, 0u, 0u};
    }
  };

  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      bf16x8 bfr[TM], afr[TN];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        bfr[tm] = *reinterpret_cast<const bf16x8*>(
            &As[buf][wm0 + tm * 16 + (lane & 15)][kk + 8 * (lane >> 4)]);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        if (DX) {
          const int j = lane & 15, grp = lane >> 4;
          const int col = wn0 + tn * 16 + 4 * (j & 3);
          const int row = kk + 8 * grp + (j >> 2);
          bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(&Ws[buf][row][col]));
          bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(&Ws[buf][row + 4][col]));
          afr[tn] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
          afr[tn] = *reinterpret_cast<const bf16x8*>(
              &Ws[buf][wn0 + tn * 16 + (lane & 15)][kk + 8 * (lane >> 4)]);
        }
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          acc[tn][tm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[tn], bfr[tm], acc[tn][tm], 0, 0, 0);
    }
  };

  // ---- main contraction: double-buffered LDS, one barrier per step
  load_step(0);
  store_step(0);
  __syncthreads();
  for (int s = 0; s < steps; ++s) {
    const int cur = s & 1;
    if (s + 1 < steps) load_step(s + 1);
    compute(cur);
    if (s + 1 < steps) store_step(cur ^ 1);
    __syncthreads();
  }

  // ---- adapter term: contraction over the rank, 64 at a time, operands staged straight to LDS
  for (int j0 = 0; j0 < g.r; j0 += kBK) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int q = tid + 256 * i;
      const int64_t row = m0 + (q >> 3);
      const int col = j0 + (q & 7) * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (row < g.M && col < g.r) {
        const f32x4* src = reinterpret_cast<const f32x4*>(g.lora_act + row * g.r + col);
        const f32x4 a = src[0], b = src[1];
        v = u32x4{pack_bf16x2(g.scale * a[0], g.scale * a[1]), pack_bf16x2(g.scale * a[2], g.scale * a[3]),
                  pack_bf16x2(g.scale * b[0], g.scale * b[1]), pack_bf16x2(g.scale * b[2], g.scale * b[3])};
      }
      *reinterpret_cast<u32x4*>(&As[0][q >> 3][(q & 7) * 8]) = v;
    }
    u32x4* dst = reinterpret_cast<u32x4*>(&Ws[0][w_row][32 * w_seg]);
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
    __syncthreads();
    compute(0);
    __syncthreads();
  }

  // ---- epilogue: lane holds 4 consecutive output columns of one row
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int64_t m = m0 + wm0 + tm * 16 + (lane & 15);
      const int64_t n = col0 + wn0 + tn * 16 + 4 * (lane >> 4);
      if (m < g.M && n < Nout) {
        const f32x4 a = acc[tn][tm];
        *reinterpret_cast<u32x2*>(g.out + m * Nout + n) =
            u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
      }
    }
  }
}

template <bool DX>
static hipError_t launch_gemm_t(const GemmArgs& g, hipStream_t stream) {
  const int64_t Nout = DX ? g.K : g.N;
  const int gx = (int)((Nout + kBN - 1) / kBN);
  if (g.M > 64) {
    const int gy = (int)((g.M + 255) / 256);
    hipLaunchKernelGGL((qlora_gemm_kernel<DX, 256>), dim3(gx, gy), dim3(256), 0, stream, g);
  } else {
    hipLaunchKernelGGL((qlora_gemm_kernel<DX, 64>), dim3(gx, 1), dim3(256), 0, stream, g);
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
