// Skinny forward of the adapted linear for a few tokens (M <= 16): the dequant-GEMV regime.
//
// "QLoRA, explained", The forward pass and gradients / The algorithm, step by step:
// y = x W~^T + s (x A^T) B^T. With M <= 16 the weight is read once and each dequantised value is
// used M times, so the kernel is bound by HBM bandwidth on the packed weight (0.52 bytes per
// value) and, behind it, by the VALU work of dequantisation. Layout of the work:
//   * rows of W (N of them) followed by the r rows of A form the "row" axis, cut into tiles of 64;
//     the k axis is cut into S splits of whole 256-column sub-chunks; (tile, split) pairs are work
//     items, taken in turn by persistent workgroups;
//   * a workgroup (4 waves) takes one item; wave w takes a contiguous quarter of the split's
//     sub-chunks and keeps the next sub-chunk's packed codes in flight in registers;
//   * lane (row = lane % 16, grp = lane / 16) dequantises the 64-value block at column
//     kb + 64 * grp of its row straight into MFMA operand registers, and the same lane holds
//     x[m = lane % 16][kb + 64 * grp ...] as the other operand, so v_mfma_f32_16x16x32_bf16
//     contracts over a permuted but consistent k order;
//   * dequantisation reads both codes of a packed byte from an LDS pair table (256 entries of two
//     fp32 codes, replicated 32 times so the 32 lanes of a half-wave read distinct banks): one
//     v_perm forms the address (byte * 256 + copy * 8), then two fp32 products with the block
//     scale and one bf16 pair conversion, giving bit for bit bf16(fl32(q[idx] * c1'));
//   * the four waves are summed in LDS in wave order and the workgroup writes one fp32 partial;
//   * skinny_epilogue_kernel sums the S partials in split order, forms u = x A^T from the A rows,
//     adds s * u B^T in fp32 and rounds y to bf16.
#include "common.h"
#include "launch.h"

namespace nf4 {

constexpr int kSub = 256;   // k columns per sub-chunk (4 lane groups x one 64-value block)

struct SkinnyArgs {
  const uint8_t* packed;
  const uint8_t* scale_q;
  const float* scale_c2;
  int64_t N, K;
  const uint16_t* x;   // [M x K] bf16
  int64_t M;
  const uint16_t* A;   // [r x K] bf16
  int r;
  int splits, sub_per_split, row_tiles;
  float* part;         // [splits][M][N + r]
};

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

// One sub-chunk of one lane in registers (raw loaded values only, so issuing the loads never
// waits for their arrival).
struct SkinnyStage {
  u32x4 p[4][2];      // [tile][half of the lane's 64-value block]
  uint32_t code[4];   // E4M3 codes of the block scales
  float c2[4];        // second-level constants
};

__constant__ uint32_t kSkinnyCodes[16] = {NF4_CODE_BITS};

__global__ __launch_bounds__(256) void skinny_fwd_kernel(const SkinnyArgs g) {
  __shared__ __attribute__((aligned(16))) f32x2 tab[256 * 32];
  __shared__ float red[4][4][64][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4;
  const int64_t rows = g.N + g.r;
  const int64_t nsub = (g.K + kSub - 1) / kSub;
  const int64_t m = lane & 15;
  const int64_t mc = min(m, g.M - 1);
  const uint32_t laneoff = (uint32_t)(lane & 31) * 8u;

  // pair table: thread t owns byte value t and writes its 32 copies (256 contiguous bytes)
  {
    const float hi = __uint_as_float(kSkinnyCodes[tid >> 4]);
    const float lo = __uint_as_float(kSkinnyCodes[tid & 15]);
    const u32x4 v = u32x4{__float_as_uint(hi), __float_as_uint(lo), __float_as_uint(hi), __float_as_uint(lo)};
    u32x4* dst = reinterpret_cast<u32x4*>(&tab[tid * 32]);
#pragma unroll
    for (int c = 0; c < 16; ++c) dst[c] = v;
  }
  __syncthreads();
  const char* tab_bytes = reinterpret_cast<const char*>(tab);

  const int items = g.row_tiles * g.splits;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int split = item / g.row_tiles;
    const int64_t row_tile0 = (int64_t)(item % g.row_tiles) * 64;
    const int64_t split_begin = (int64_t)split * g.sub_per_split;
    const int64_t split_end = min(nsub, split_begin + g.sub_per_split);
    const int64_t per_wave = (split_end - split_begin + 3) / 4;
    const int64_t sub_begin = split_begin + wave * per_wave;
    const int64_t sub_end = min(split_end, sub_begin + per_wave);
    bool nf4_tile[4], live_tile[4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
      const int64_t first = row_tile0 + tn * 16;
      nf4_tile[tn] = first < g.N;
      live_tile[tn] = first < rows;
    }
    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // branch-free loads: row and column are clamped into range; data of rows or columns out of
    // range is never used (its tile is not an NF4 tile, or its k range is past K and masked)
    auto load_stage = [&](int64_t sub, SkinnyStage& st) {
      const int64_t kk = min(sub * kSub + 64 * grp, g.K - 64);
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) {
        const int64_t row = min(row_tile0 + tn * 16 + (lane & 15), g.N - 1);
        const int64_t e = row * g.K + kk;
        const u32x4* src = reinterpret_cast<const u32x4*>(g.packed + e / 2);
        st.p[tn][0] = __builtin_nontemporal_load(src);
        st.p[tn][1] = __builtin_nontemporal_load(src + 1);
        st.code[tn] = g.scale_q[e / kBlock];
        st.c2[tn] = g.scale_c2[e / kBlock / kGroup];
      }
    };

    auto process = [&](int64_t sub, const SkinnyStage& st) {
      const int64_t kk0 = sub * kSub + 64 * grp;
      const bool kvalid = kk0 < g.K;
      const int64_t kk = min(kk0, g.K - 64);
      bf16x8 b[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        b[j] = *reinterpret_cast<const bf16x8*>(g.x + mc * g.K + kk + 8 * j);
        if (!kvalid || m >= g.M) b[j] = bf16x8{};
      }
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) {
        if (!live_tile[tn]) continue;
        uint32_t a[8][4];
        if (nf4_tile[tn]) {
          const float c1p = __fmul_rn(e4m3_decode(st.code[tn]), st.c2[tn]);
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const uint32_t word = st.p[tn][h][d];
#pragma unroll
              for (int bb = 0; bb < 4; ++bb) {
                // byte bb of the word holds values 8 * (4h + d) + 2bb (high nibble) and + 1
                const uint32_t off = __builtin_amdgcn_perm(word, laneoff, 0x0C0C0000u | ((4u + bb) << 8));
                const f32x2 qv = *reinterpret_cast<const f32x2*>(tab_bytes + off);
                a[4 * h + d][bb] = pack_bf16x2(__fmul_rn(qv[0], c1p), __fmul_rn(qv[1], c1p));
              }
            }
        } else {
          const int64_t j = row_tile0 + tn * 16 + (lane & 15) - g.N;
          const int64_t jc = min(j, (int64_t)g.r - 1);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            u32x4 v = *reinterpret_cast<const u32x4*>(g.A + jc * g.K + kk + 8 * i);
            if (j >= g.r) v = u32x4{0u, 0u, 0u, 0u};
            a[i][0] = v[0]; a[i][1] = v[1]; a[i][2] = v[2]; a[i][3] = v[3];
          }
        }
        if (!kvalid) {
#pragma unroll
          for (int i = 0; i < 8; ++i) a[i][0] = a[i][1] = a[i][2] = a[i][3] = 0u;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const u32x4 av = u32x4{a[i][0], a[i][1], a[i][2], a[i][3]};
          acc[tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), b[i],
                                                            acc[tn], 0, 0, 0);
        }
      }
    };

    // two register stages: while sub-chunk i is dequantised, sub-chunk i+1 is in flight
    SkinnyStage s0, s1;
    if (sub_begin < sub_end) {
      load_stage(sub_begin, s0);
      for (int64_t sub = sub_begin; sub < sub_end; sub += 2) {
        load_stage(min(sub + 1, sub_end - 1), s1);
        process(sub, s0);
        if (sub + 1 >= sub_end) break;
        load_stage(min(sub + 2, sub_end - 1), s0);
        process(sub + 1, s1);
      }
    }

    // acc[tn][i]: row = tile row tn*16 + 4*grp + i, column m = lane % 16
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][tn][lane][i] = acc[tn][i];
    __syncthreads();
    // 64 rows x 16 columns per item; thread t takes (row = t / 4, m = 4 * (t % 4) .. +3)
    const int rloc = tid >> 2, tq = rloc >> 4, rin = rloc & 15;
    const int64_t row = row_tile0 + rloc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int mm = 4 * (tid & 3) + q;
      const int ln = (rin >> 2) * 16 + mm, ii = rin & 3;
      const float v = ((red[0][tq][ln][ii] + red[1][tq][ln][ii]) + red[2][tq][ln][ii]) + red[3][tq][ln][ii];
      if (mm < g.M && row < rows) g.part[((int64_t)split * g.M + mm) * rows + row] = v;
    }
    __syncthreads();
  }
}

// y[m][n] = bf16(sum_s part[s][m][n] + scale * sum_j u[m][j] B[n][j]),  u[m][j] = sum_s part[s][m][N + j].
// Workgroup = 64 columns; it rebuilds u (M x r, at most 16 x 128) in LDS from the adapter-row
// partials and stages its columns of B; thread t takes column t % 64 and tokens t / 64, +4, ...
__global__ __launch_bounds__(256) void skinny_epilogue_kernel(const float* __restrict__ part, int splits,
                                                              int64_t M, int64_t N, int r,
                                                              const uint16_t* __restrict__ B, float scale,
                                                              float* __restrict__ u_out,
                                                              uint16_t* __restrict__ y) {
  __shared__ float us[16][128];
  __shared__ float bs[128][64 + 1];
  const int64_t rows = N + r;
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  for (int idx = threadIdx.x; idx < M * r; idx += 256) {
    const int mm = idx / r, j = idx % r;
    float s = 0.f;
    for (int sp = 0; sp < splits; ++sp) s += part[((int64_t)sp * M + mm) * rows + N + j];
    us[mm][j] = s;
    if (blockIdx.x == 0) u_out[(int64_t)mm * r + j] = s;
  }
  for (int idx = threadIdx.x; idx < 64 * r; idx += 256) {
    const int nl = idx / r, j = idx % r;
    bs[j][nl] = (n0 + nl < N) ? __uint_as_float((uint32_t)B[(n0 + nl) * r + j] << 16) : 0.f;
  }
  __syncthreads();
  const int nl = threadIdx.x & 63;
  const int64_t n = n0 + nl;
  if (n >= N) return;
  for (int mm = threadIdx.x >> 6; mm < M; mm += 4) {
    float s = 0.f;
    for (int sp = 0; sp < splits; ++sp) s += part[((int64_t)sp * M + mm) * rows + n];
    float l = 0.f;
    for (int j = 0; j < r; ++j) l = fmaf(us[mm][j], bs[j][nl], l);
    const float v = s + scale * l;
    y[mm * N + n] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu);
  }
}

bool skinny_eligible(int64_t M) { return M >= 1 && M <= 16; }

void skinny_plan(int64_t N, int64_t K, int r, int* splits, int* sub_per_split, int* row_tiles) {
  *row_tiles = (int)((N + r + 63) / 64);
  const int64_t nsub = (K + kSub - 1) / kSub;
  int64_t want = (1024 + *row_tiles - 1) / *row_tiles;
  int64_t cap = nsub / 16;       // keep at least 16 sub-chunks (four per wave) per split
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  *sub_per_split = (int)((nsub + want - 1) / want);
  *splits = (int)((nsub + *sub_per_split - 1) / *sub_per_split);
}

size_t skinny_workspace_floats(int64_t M, int64_t N, int64_t K, int r) {
  int s, spp, rt;
  skinny_plan(N, K, r, &s, &spp, &rt);
  return (size_t)s * (size_t)M * (size_t)(N + r);
}

hipError_t launch_skinny_fwd(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                             int64_t N, int64_t K, const uint16_t* x, int64_t M, const uint16_t* A,
                             const uint16_t* B, int r, float scale, float* part, float* u_out,
                             uint16_t* y, hipStream_t stream) {
  int splits, spp, row_tiles;
  skinny_plan(N, K, r, &splits, &spp, &row_tiles);
  SkinnyArgs g{packed, scale_q, scale_c2, N, K, x, M, A, r, splits, spp, row_tiles, part};
  const int items = row_tiles * splits;
  const int grid = items < 512 ? items : 512;   // two 80 KB workgroups per CU
  hipLaunchKernelGGL(skinny_fwd_kernel, dim3((unsigned)grid), dim3(256), 0, stream, g);
  hipLaunchKernelGGL(skinny_epilogue_kernel, dim3((unsigned)((N + 63) / 64)), dim3(256), 0, stream,
                     part, splits, M, N, r, B, scale, u_out, y);
  return hipGetLastError();
}

}  // namespace nf4
