// Fused dequantise + bf16 MFMA GEMMs of the adapted linear (gfx950).
//
// "QLoRA, explained", The forward pass and gradients / The algorithm, step by step:
//   forward   y  = X W~^T + s (X A^T) B^T            (contraction over K)
//   backward  dX = dY W~  + s (dY B) A               (contraction over N; W is read again)
// W~ never exists in HBM: the packed NF4 codes of a tile are dequantised into LDS with a per-block
// bf16 lookup table and fed to bf16 MFMAs. The adapter term rides on the same accumulators as extra
// contraction steps: operands bf16(s * u) with B (forward) or bf16(s * v) with A (backward), where
// u = X A^T and v = dY B come from the LoRA kernels.
//
// Workgroup = 16 waves on a BM x 128 output tile, contraction in steps of 64, three roles:
//   * waves 0-7 (consumers) only read LDS and issue v_mfma_f32_32x32x16_bf16. Two of them share
//     each SIMD, so one issues MFMAs while the other waits on its LDS reads;
//   * waves 8-11 (dequantisers) turn the packed weight, its scale codes and second-level constants
//     of a step (already in LDS) into the bf16 W tile: VALU work and LDS accesses only;
//   * waves 12-15 (loaders) issue every global load as a 16-byte LDS-DMA buffer load: activation
//     tiles one step ahead, packed weight tiles three steps ahead. The address unit takes a few tens
//     of cycles per such load, so these waves spend most of their time waiting to issue; keeping
//     that off the other waves' instruction streams is why they exist.
// The roles meet at one workgroup barrier per phase. In phase q the loaders fetch activations of
// step q+1 and packed weights of step q+3, the dequantisers build the W tile of step q (from
// registers) while reading the packed words of step q+1, and the consumers multiply step q-1.
// LDS holds three activation stages, two W stages and four packed weight stages.
//
// Activation rows are 128 bytes in LDS (no padding, as DMA writes 64 lanes x 16 contiguous bytes);
// the 16-byte chunk c of row r sits at slot c ^ ((r >> 1) & 7), which keeps the 16-lane groups of a
// fragment read on distinct banks. The W tile is stored [row of W][column of W] (K contiguous) for
// both directions: the forward reads it row-wise with ds_read_b128, the backward column-wise with
// ds_read_b64_tr_b16 (within 16 lanes, lane j receives element j%4 of the 8-byte rows addressed by
// lanes j/4, j/4+4, j/4+8 and j/4+12).
//
// Ragged edges need no per-element tests: buffer loads past the end of a tile's records return
// zeros (activation rows past M, weight rows past N, their codes and constants), and the one
// partial contraction step of the backward (N % 64 != 0) points its missing activation chunks past
// the records. Weight rows past N dequantise to exact zeros there (code 0 and constant 0); in the
// forward they only feed output columns that are not stored.
//
// Split contraction (ksplit > 1, forward only): when a launch would leave most CUs idle (few
// output tiles), each tile's contraction is cut into ksplit ranges taken by separate workgroups.
// A tile's time is set by its number of steps (a step costs the dequantisers' work on one W tile,
// whatever the tile's height), so halving the steps per workgroup halves it. Each range writes
// fp32 partial sums; gemm_ksum_kernel adds them in range order and rounds to bf16. The adapter
// steps ride with the last range. The same cut applied to the last, partial round of tiles only
// (tail mode, forward and dX) keeps that round from leaving most CUs idle; see GemmPlan.
//
// With F32S the weight keeps one fp32 absmax per block instead of double-quantised scales (the
// baseline of "QLoRA, explained", Double quantisation): the loaders bring that scale where they
// bring the E4M3 code word otherwise, there is no second-level constant, and c1' is the scale.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace nf4 {

// One weight of a grouped launch over several adapted linears that share their input x (a layer's
// query, key and value projections, or its gate and up projections). Forward: the column tiles run
// over the weights in turn (y_i = x W~_i^T + ...). dX: each weight's tiles in turn, every linear
// with its own dY_i and dX_i (dX_i = dY_i W~_i + ...).
struct GemmWeight {
  const uint8_t* packed;
  const uint8_t* scale_q;
  const float* scale_c2;
  const float* absmax;
  int64_t N;
  const uint16_t* act;      // dY of this linear [M x N] (dX only)
  const float* lora_act;    // u [M x r] (forward) or v [M x r] (dX) of this linear
  const uint16_t* lora_w;   // B [N x r] (forward) or A [r x K] (dX) of this linear
  uint16_t* out;            // y [M x N] or dX [M x K] of this linear
  int tile0;                // forward: its first column tile in the group
};
constexpr int kMaxGroup = 4;

struct GemmArgs {
  const uint8_t* packed;
  const uint8_t* scale_q;
  const float* scale_c2;
  const float* absmax;      // fp32 scales (F32S) instead of scale_q and scale_c2
  int64_t N, K;             // W is N x K
  const uint16_t* act;      // X [M x K] (forward) or dY [M x N] (backward), bf16
  int64_t M;
  const float* lora_act;    // u [M x r] (forward) or v [M x r] (backward), fp32
  const uint16_t* lora_w;   // B [N x r] (forward) or A [r x K] (backward), bf16
  int r;
  float scale;
  uint16_t* out;            // y [M x N] (forward) or dX [M x K] (backward), bf16
  int ksplit;               // contraction ranges of every tile (1: none)
  float* part;              // ksplit x M x Nout fp32 partial sums when ksplit > 1; the tail's
                            // pieces otherwise (tail_split x tail_tiles x BM x kBN, tile-major)
  int whole_tiles;          // tail mode (tail_tiles > 0): tiles 0 .. whole_tiles - 1 whole,
  int tail_tiles;           //   the last tail_tiles tiles cut into tail_split contraction ranges
  int tail_split;
  Codes codes;              // the values the 4-bit indices select
  int nw;                   // grouped forward: weights in w (1: the fields above are the weight)
  int gx_total;             //   column tiles of all of them
  GemmWeight w[kMaxGroup];
};

constexpr int kBN = 128;        // output columns per tile
constexpr int kBK = 64;         // contraction per step
constexpr int kXStages = 3;     // activation stages in LDS
constexpr int kPStages = 4;     // packed weight stages in LDS
constexpr int kThreads = 1024;  // 8 consumer + 4 dequantiser + 4 loader waves

// Weight wi of a grouped launch into g (uniform per workgroup; a select per field keeps the kernel
// arguments out of private memory).
template <bool DX>
__device__ __forceinline__ void use_weight(GemmArgs& g, const GemmArgs& ga, int wi) {
#pragma unroll
  for (int i = 0; i < kMaxGroup; ++i) {
    if (i == wi) {
      g.packed = ga.w[i].packed;
      g.scale_q = ga.w[i].scale_q;
      g.scale_c2 = ga.w[i].scale_c2;
      g.absmax = ga.w[i].absmax;
      g.N = ga.w[i].N;
      if (DX) g.act = ga.w[i].act;
      g.lora_act = ga.w[i].lora_act;
      g.lora_w = ga.w[i].lora_w;
      g.out = ga.w[i].out;
    }
  }
}

// The weight of a grouped forward that owns global column tile gcol, and the tile's first column
// within it.
__device__ __forceinline__ void select_weight(GemmArgs& g, const GemmArgs& ga, int gcol, int64_t& col0) {
  int wi = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i)
    if (i < ga.nw && gcol >= ga.w[i].tile0) wi = i;
  use_weight<false>(g, ga, wi);
#pragma unroll
  for (int i = 0; i < kMaxGroup; ++i)
    if (i == wi) col0 = (int64_t)(gcol - ga.w[i].tile0) * kBN;
}

template <bool DX>
struct WTile {
  static constexpr int rows = DX ? kBK : kBN;            // contraction rows (DX) or output rows
  // forward: 144-byte rows put 16 consecutive rows in 16 distinct 16-byte slots of the 64-bank
  // (256-byte) LDS. dX: unpadded 256-byte rows with the 16-byte chunks swizzled (wswz)
  static constexpr int pitch = DX ? kBN : kBK + 8;
  static constexpr int segs = DX ? kBN / 32 : kBK / 32;  // 32-value segments per row
};

template <int BM>
struct Waves {  // consumer layout: waves_m x waves_n waves, each on a WM x WN sub-tile
  static constexpr int waves_m = BM == 64 ? 2 : 4;
  static constexpr int waves_n = 8 / waves_m;
  static constexpr int WM = BM / waves_m, WN = kBN / waves_n;
  static constexpr int TM = WM / 32, TN = WN / 32;
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
// The LDS words a dequantiser thread expands in one step: its 32-value packed chunk, the word
// holding its block's scale code and the block's second-level constant.
struct StepWords {
  u32x4 wq;
  uint32_t cw, c2;
};

// Element offset of (row, col) within a row of the dX W tile: chunk k (8 values, 16 bytes) of row r
// sits at chunk k ^ 5 (r & 3). A transpose read (lanes 0-31: four rows r..r+3, r % 4 == 0, times
// four aligned chunks) then meets 16 distinct chunk positions (the XOR's upper two bits differ per
// row), and so does a dequantiser store (four rows times one chunk in each of four 64-byte
// segments: the XOR's lower two bits differ per row). With padded 288-byte rows instead, the reads
// overlapped in the bank window and 17 % of the GEMM's cycles stalled on bank conflicts.
__device__ __forceinline__ int wswz(int row, int col) {
  return ((((col >> 3) ^ (5 * (row & 3))) << 3) | (col & 7));
}

// Swap with the neighbouring lane (quad_perm [1,0,3,2]).
__device__ __forceinline__ uint32_t swap_pair(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}

template <bool DX, int BM, bool F32S>
__global__ __launch_bounds__(kThreads) void qlora_gemm_kernel(const GemmArgs ga) {
  using WT = WTile<DX>;
  using CW = Waves<BM>;
  constexpr int TM = CW::TM, TN = CW::TN;
  constexpr int NX = BM / 32;                 // activation DMA loads per loader wave per phase
  static_assert(NX <= 8, "activation DMA offsets");
  constexpr int XSTAGE = BM * kBK;            // elements per activation stage

  __shared__ __attribute__((aligned(16))) uint16_t Xs[kXStages * XSTAGE];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][WT::rows][WT::pitch];
  __shared__ __attribute__((aligned(16))) u32x4 Ps[kPStages][256];     // packed weight chunks
  __shared__ __attribute__((aligned(16))) uint32_t Cs[kPStages][256];  // words holding scale codes
  __shared__ __attribute__((aligned(16))) float Gs[kPStages][256];     // second-level constants

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  GemmArgs g = ga;                          // a grouped launch's workgroup swaps in its weight
  // column tiles (of the whole group in a grouped forward; of each weight's dX, all of width K)
  const int gx = (!DX && ga.nw > 1) ? ga.gx_total : (int)(((DX ? g.K : g.N) + kBN - 1) / kBN);

  // Tile coordinates. Workgroups are dealt round-robin over the 8 XCDs (workgroup i to XCD i % 8,
  // in order of i), so each XCD gets a contiguous run of tiles that share an activation row block.
  // Uniform split: the contraction range is the slowest index, so the ranges of a tile go to
  // different XCDs. Tail mode (the tiles past the last whole round of the CUs cut into ranges, so
  // that the last round is full): each XCD first takes its share of the whole tiles, then its
  // share of the tail's pieces.
  const int total = gridDim.x * gridDim.y;
  const int bid = blockIdx.x + gridDim.x * blockIdx.y;
  int tile, split = 0, nsplit = g.ksplit, tail_r = 0;
  if (g.tail_tiles > 0) {
    const int xcd = bid & 7, k = bid >> 3;
    const int wx = g.whole_tiles >> 3, px = (g.tail_tiles * g.tail_split) >> 3;
    if (k < wx) {
      tile = xcd * wx + k;
      nsplit = 1;
    } else {
      const int piece = xcd * px + (k - wx);
      tail_r = piece / g.tail_split;
      split = piece % g.tail_split;
      tile = g.whole_tiles + tail_r;
      nsplit = g.tail_split;
    }
  } else if (DX && ga.nw > 1) {
    // grouped dX: T tiles per weight; each XCD takes a contiguous run of every weight's tiles in
    // turn (the longest contraction first, as the caller orders them), so the XCDs get equal work
    const int T = total / ga.nw;
    int wi;
    if ((T & 7) == 0) {
      const int xcd = bid & 7, k = bid >> 3, t8 = T >> 3;
      wi = k / t8;
      tile = xcd * t8 + k % t8;
    } else {
      wi = bid / T;
      tile = bid % T;
    }
    use_weight<true>(g, ga, wi);
  } else {
    int lin = bid;
    if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
    const int tiles = total / g.ksplit;
    split = lin / tiles;
    tile = lin % tiles;
  }
  int64_t col0 = (int64_t)(tile % gx) * kBN;
  const int64_t m0 = (int64_t)(tile / gx) * BM;
  if (!DX && ga.nw > 1) select_weight(g, ga, tile % gx, col0);
  const int64_t Lc = DX ? g.N : g.K;       // contraction length
  const int64_t Nout = DX ? g.K : g.N;     // output columns

  const int main_total = (int)((Lc + kBK - 1) / kBK);
  const int per_split = (main_total + nsplit - 1) / nsplit;
  const int T0 = split * per_split;        // first contraction step of this range
  const int main_steps = min(per_split, main_total - T0);
  const int lora_steps = split == nsplit - 1 ? (g.r + kBK - 1) / kBK : 0;
  const int steps = main_steps + lora_steps;
  const uint32_t kb = (uint32_t)(g.K / kBlock);   // blocks per row of W

  if (wave >= 12) {
    // ================================================================ loaders
    const int lw = wave - 12;
    // ---- activation tile: instruction j of wave lw fills 16-byte slots lw * 2BM + 64 j + lane of
    //      the stage; slot (row, s) holds logical chunk s ^ ((row >> 1) & 7)
    const int64_t rows_valid = min(g.M - m0, (int64_t)BM);
    uint32_t xoff[8];   // NX <= 8 entries used (a fixed size: lambdas that capture an array whose
                        // size depends on a template parameter lose the kernel's host-side stub)
#pragma unroll
    for (int j = 0; j < NX; ++j) {
      const int slot = lw * 2 * BM + j * 64 + lane;
      const int row = slot >> 3, c = (slot & 7) ^ ((row >> 1) & 7);
      xoff[j] = (uint32_t)row * (uint32_t)(Lc * 2) + (uint32_t)c * 16u;
    }
    // `full`: the step is known to be a whole one (every step but the last), so the loop that
    // issues those carries no per-chunk selects
    auto issue_x = [&](int t, bool full) {
      const int tg = t + T0;
      const uint16_t* base = g.act + m0 * Lc + (int64_t)tg * kBK;
      const int nrec = (int)(rows_valid * Lc * 2 - (int64_t)tg * kBK * 2);
      __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nrec, kRsrcFlags);
      uint16_t* dst = Xs + (t % kXStages) * XSTAGE + (lw * 2 * BM) * 8;
      if (full || (int64_t)(tg + 1) * kBK <= Lc) {
#pragma unroll
        for (int j = 0; j < NX; ++j) {
          const uint32_t off = xoff[j];
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + j * 64 * 8), 16, off, 0, 0, 0);
        }
      } else {   // a backward's last step with N % 64 != 0: chunks past N read zeros
        const int valid_chunks = (int)(Lc - (int64_t)tg * kBK) / 8;
#pragma unroll
        for (int j = 0; j < NX; ++j) {
          const int slot = lw * 2 * BM + j * 64 + lane;
          const int row = slot >> 3, c = (slot & 7) ^ ((row >> 1) & 7);
          const uint32_t off = c < valid_chunks ? xoff[j] : kOutOfRange;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + j * 64 * 8), 16, off, 0, 0, 0);
        }
      }
    };

    // ---- packed weight tile: slot lw * 64 + lane is the 32-value chunk the dequantiser thread of
    //      the same index expands (row w_row, segment w_seg of the W tile)
    const int pslot = lw * 64 + lane;
    const int w_row = pslot / WT::segs, w_seg = pslot % WT::segs;
    const uint32_t wp_off = (uint32_t)w_row * (uint32_t)(g.K / 2) + (uint32_t)w_seg * 16u;
    const int64_t nblocks = g.N * (g.K / kBlock);
    __amdgpu_buffer_rsrc_t rs_q = F32S
        ? __builtin_amdgcn_make_buffer_rsrc((void*)g.absmax, (short)0, (int)(nblocks * 4), kRsrcFlags)
        : __builtin_amdgcn_make_buffer_rsrc((void*)g.scale_q, (short)0, (int)nblocks, kRsrcFlags);
    __amdgpu_buffer_rsrc_t rs_c2 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.scale_c2, (short)0, (int)(((nblocks + kGroup - 1) / kGroup) * 4), kRsrcFlags);
    // scales: forward, one block per W row and step (rows 0-63 by waves 0/2, 64-127 by 1/3: the
    // word holding the code, then the constant); backward, two blocks per W row (wave 0: the 16
    // bytes from the aligned word holding both codes, wave 1: 16 bytes of constants)
    const int srow = DX ? lane : (lw & 1) * 64 + lane;
    const uint32_t sb0 = DX ? (uint32_t)srow * kb + (uint32_t)(col0 / kBlock) : (uint32_t)(col0 + srow) * kb;
    const uint32_t sb_step = DX ? (uint32_t)kBK * kb : 1u;
    auto issue_p = [&](int t) {
      const int tg = t + T0;
      const uint8_t* base;
      int64_t nrec;
      if (DX) {
        base = g.packed + (int64_t)tg * kBK * (g.K / 2) + col0 / 2;
        nrec = (g.N - (int64_t)tg * kBK) * (g.K / 2) - col0 / 2;
      } else {
        base = g.packed + col0 * (g.K / 2) + (int64_t)tg * (kBK / 2);
        nrec = min(g.N - col0, (int64_t)kBN) * (g.K / 2) - (int64_t)tg * (kBK / 2);
      }
      __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)nrec, kRsrcFlags);
      const int ps = t % kPStages;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(&Ps[ps][lw * 64]), 16, wp_off, 0, 0, 0);
      const uint32_t b = sb0 + (uint32_t)tg * sb_step;
      if (F32S) {
        // forward: the block's scale for rows 0-63 (wave 0) and 64-127 (wave 1); backward: the
        // row's two blocks, the first by wave 0 and the second by wave 1
        if (DX) {
          if (lw == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_q, (lds_void*)(&Cs[ps][0]), 4, b * 4u, 0, 0, 0);
          else if (lw == 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_q, (lds_void*)(&Gs[ps][0]), 4, (b + 1u) * 4u, 0, 0, 0);
        } else if (lw < 2) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_q, (lds_void*)(&Cs[ps][(lw & 1) * 64]), 4, b * 4u, 0, 0, 0);
        }
      } else if (DX) {
        if (lw == 0) {
          const uint32_t off = b & ~3u;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_q, (lds_void*)(&Cs[ps][0]), 16, off, 0, 0, 0);
        } else if (lw == 1) {
          const uint32_t off = (b >> 8) * 4u;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_c2, (lds_void*)(&Gs[ps][0]), 16, off, 0, 0, 0);
        }
      } else {
        if (lw < 2) {
          const uint32_t off = b & ~3u;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_q, (lds_void*)(&Cs[ps][(lw & 1) * 64]), 4, off, 0, 0, 0);
        } else {
          const uint32_t off = (b >> 8) * 4u;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_c2, (lds_void*)(&Gs[ps][(lw & 1) * 64]), 4, off, 0, 0, 0);
        }
      }
    };

    // ---- schedule. Phase q issues the activations of step q+1, then the packed weights of step
    // q+3, and waits until everything issued in phase q-1 has landed: the loads issued in phase q
    // are the only ones allowed to stay in flight, and vector-memory loads complete in issue order.
    // The packed weights of a step therefore sit in LDS one phase before they are expanded, which
    // lets the dequantisers read them a phase ahead.
    const bool two_p = (!DX && !F32S) || lw < 2;   // issue_p makes two loads (chunk + a scale word)
    issue_x(0, false);
    issue_p(0);
    if (main_steps > 1) issue_p(1);
    if (main_steps > 2) issue_p(2);
    wait_vmcnt<0>();
    lds_barrier();
    auto phase = [&](int q, bool full) {
      const bool more_x = q + 1 < main_steps, more_p = q + 3 < main_steps;
      if (more_x) issue_x(q + 1, full);
      if (more_p) issue_p(q + 3);
      if (more_p) {
        if (two_p) wait_vmcnt<NX + 2>();
        else wait_vmcnt<NX + 1>();
      } else if (more_x) {
        wait_vmcnt<NX>();
      } else {
        wait_vmcnt<0>();
      }
      lds_barrier();
    };
    int q = 0;
    for (; q + 2 < main_steps; ++q) phase(q, true);   // step q + 1 is not the last one
    for (; q <= steps; ++q) phase(q, false);
    return;
  }

  if (wave >= 8) {
    // ================================================================ dequantisers
    const int dt = tid - 512;   // 0..255: the packed chunk of this thread
    const int w_row = dt / WT::segs, w_seg = dt % WT::segs;
    // ---- dequantisation with a lookup table shared by the lane pair that holds one block: lane
    // parity h computes the bf16 products of codes 8h .. 8h+7 and receives the other half from its
    // neighbour. Odd lanes flip bit 3 of every index so that "own half" is entries 0..7 for both.
    const uint32_t h = lane & 1;
    float qv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = h ? g.codes.v[8 + i] : g.codes.v[i];
    const uint32_t hx = h ? 0x88888888u : 0u, hx4 = hx >> 4;
    // block index of this thread's chunk at step t: b0 + t * b_step; where its code and constant
    // sit in the scale stages
    const uint32_t b0 = DX ? (uint32_t)w_row * kb + (uint32_t)((col0 + 32 * w_seg) / kBlock)
                           : (uint32_t)(col0 + w_row) * kb;
    const uint32_t b_step = DX ? (uint32_t)kBK * kb : 1u;
    const uint32_t rb0 = DX ? (uint32_t)w_row * kb + (uint32_t)(col0 / kBlock) : b0;   // the row's first block
    // The LDS words of step t are read one phase before they are expanded (they landed a phase
    // earlier still), so the reads wait behind the consumers' fragment reads off the critical path.
    // Only raw loaded words cross the phase: anything computed from them would make the compiler
    // wait for the reads in the phase that issues them.
    auto fetch = [&](int t) {
      const int ps = t % kPStages;
      StepWords w;
      w.wq = Ps[ps][dt];
      if (F32S) {
        w.cw = DX && (w_seg >> 1) ? __float_as_uint(Gs[ps][w_row]) : Cs[ps][w_row];
        w.c2 = 0u;
      } else if (DX) {
        const uint32_t b = b0 + (uint32_t)(t + T0) * b_step, rb = rb0 + (uint32_t)(t + T0) * b_step;
        const uint32_t byte = (rb & 3u) + (uint32_t)(w_seg >> 1);     // within the row's 16 bytes
        w.cw = Cs[ps][w_row * 4 + (int)(byte >> 2)];
        w.c2 = __float_as_uint(Gs[ps][w_row * 4 + (int)((b >> 8) - (rb >> 8))]);
      } else {
        w.cw = Cs[ps][w_row];
        w.c2 = __float_as_uint(Gs[ps][w_row]);
      }
      return w;
    };
    auto dequant = [&](int t, const StepWords& sw) {
      const u32x4 wq = sw.wq;
      uint32_t shift;   // byte of the code within its word
      if (DX) {
        const uint32_t rb = rb0 + (uint32_t)(t + T0) * b_step;
        shift = (((rb & 3u) + (uint32_t)(w_seg >> 1)) & 3u) * 8u;
      } else {
        shift = ((b0 + (uint32_t)(t + T0)) & 3u) * 8u;
      }
      const uint32_t word = sw.cw >> shift;
      const float c1p = F32S ? __uint_as_float(sw.cw)
                             : __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)word, 0), __uint_as_float(sw.c2));
      uint32_t pp[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) pp[k] = pack_bf16x2(__fmul_rn(qv[2 * k], c1p), __fmul_rn(qv[2 * k + 1], c1p));
      BlockLut L;
      L.lo[0] = __builtin_amdgcn_perm(pp[1], pp[0], 0x06040200u);
      L.lo[1] = __builtin_amdgcn_perm(pp[3], pp[2], 0x06040200u);
      L.hi[0] = __builtin_amdgcn_perm(pp[1], pp[0], 0x07050301u);
      L.hi[1] = __builtin_amdgcn_perm(pp[3], pp[2], 0x07050301u);
      L.lo[2] = swap_pair(L.lo[0]);
      L.lo[3] = swap_pair(L.lo[1]);
      L.hi[2] = swap_pair(L.hi[0]);
      L.hi[3] = swap_pair(L.hi[1]);
      // all 32 values are expanded before any is stored: an LDS write cannot issue while the
      // consumers' fragment reads fill the LDS queue, and a stalled write would hold up the
      // arithmetic behind it
      uint32_t d[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t p = wq[i];
        const uint32_t odd = (p ^ hx) & 0x0F0F0F0Fu;           // elements 1,3,5,7
        // elements 0,2,4,6: ((p >> 4) ^ hx4) & 0x0F0F0F0F as one v_bitop3 (truth table 0x28)
        const uint32_t even = __builtin_amdgcn_bitop3_b32(p >> 4, hx4, 0x0F0F0F0Fu, 0x28);
        const uint32_t s0 = __builtin_amdgcn_perm(odd, even, 0x05010400u);  // elements 0..3
        const uint32_t s1 = __builtin_amdgcn_perm(odd, even, 0x07030602u);  // elements 4..7
        lut4(L, s0, d[i][0], d[i][1]);
        lut4(L, s1, d[i][2], d[i][3]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (DX) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x4*>(&Ws[t & 1][w_row][wswz(w_row, 32 * w_seg + 8 * i)]) =
              u32x4{d[i][0], d[i][1], d[i][2], d[i][3]};
      } else {
        u32x4* dst = reinterpret_cast<u32x4*>(&Ws[t & 1][w_row][32 * w_seg]);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = u32x4{d[i][0], d[i][1], d[i][2], d[i][3]};
      }
    };

    // ---- adapter steps: bf16(s * u) (or v) into the activation stage, B (or A) into the W stage
    auto store_lora = [&](int t) {
      const int j0 = (t - main_steps) * kBK;
      uint16_t* xs = Xs + (t % kXStages) * XSTAGE;
#pragma unroll
      for (int i = 0; i < BM * 8 / 256; ++i) {
        const int q = dt + 256 * i;
        const int row = q >> 3, c = q & 7;
        const int64_t m = m0 + row;
        const int j = j0 + c * 8;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (m < g.M && j < g.r) {
          const f32x4* src = reinterpret_cast<const f32x4*>(g.lora_act + m * g.r + j);
          const f32x4 a = src[0], b = src[1];
          const float sc = g.scale;
          v = u32x4{pack_bf16x2(sc * a[0], sc * a[1]), pack_bf16x2(sc * a[2], sc * a[3]),
                    pack_bf16x2(sc * b[0], sc * b[1]), pack_bf16x2(sc * b[2], sc * b[3])};
        }
        *reinterpret_cast<u32x4*>(xs + row * kBK + ((c ^ ((row >> 1) & 7)) * 8)) = v;
      }
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
        const int wc = DX ? wswz(w_row, 32 * w_seg + 8 * i) : 32 * w_seg + 8 * i;
        *reinterpret_cast<u32x4*>(&Ws[t & 1][w_row][wc]) = v;
      }
    };

    // one phase: expand step q's words (read a phase ago) while reading step q + 1's into `nxt`;
    // the loop below alternates two sets of words, so none is copied from one phase to the next
    auto phase = [&](int q, const StepWords& cur, StepWords& nxt) {
      if (q < main_steps) {
        if (q + 1 < main_steps) nxt = fetch(q + 1);
        dequant(q, cur);
      } else if (q < steps) {
        store_lora(q);
      }
      lds_barrier();
    };
    lds_barrier();
    StepWords wa = fetch(0), wb = wa;
    for (int q = 0; q <= steps; q += 2) {   // steps + 1 phases, one barrier each
      phase(q, wa, wb);
      if (q + 1 <= steps) phase(q + 1, wb, wa);
    }
    return;
  }

  // ================================================================ consumers
  // v_mfma_f32_32x32x16_bf16: operand lane l holds row/column l % 32 and contraction 8 * (l / 32)
  // .. +7; the result lane l holds column l % 32 and rows 8 * (q / 4) + 4 * (l / 32) + q % 4 for
  // register q. The weight operand is the row side, so a lane ends up with four consecutive output
  // columns of one activation row.
  const int cw = tid >> 6;
  const int wm0 = (cw % CW::waves_m) * CW::WM, wn0 = (cw / CW::waves_m) * CW::WN;
  f32x16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // activation fragment of chunk pair kk: row wm0 + tm*32 + lane%32 (a multiple of 32 plus
  // lane%32, so its swizzle is ((lane % 32) >> 1) & 7), logical chunk 2 kk + lane/32
  int xaddr[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    xaddr[kk] = (wm0 + (lane & 31)) * kBK + (((2 * kk + (lane >> 5)) ^ ((lane >> 1) & 7)) * 8);

  // step s reads activation stage s % 3 and W buffer s % 2, passed as compile-time constants so
  // that every LDS address is a fixed offset from a per-lane base
  auto compute = [&](auto xs_t, auto wb_t) {
    constexpr int XS = decltype(xs_t)::value, wb = decltype(wb_t)::value;
    const uint16_t* xs = Xs + XS * XSTAGE;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 afr[TN], bfr[TM];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        bfr[tm] = *reinterpret_cast<const bf16x8*>(xs + xaddr[kk] + tm * 32 * kBK);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        if (DX) {
          // two 16-lane transpose loads per operand: lane group g16 covers output columns
          // (g16 & 1) * 16 .. +15 and contraction rows 8 * (g16 >> 1) .. +7
          const int j = lane & 15, g16 = lane >> 4;
          const int row = kk * 16 + (g16 >> 1) * 8 + (j >> 2);
          const int col = wswz(row, wn0 + tn * 32 + (g16 & 1) * 16 + 4 * (j & 3));   // rows row, row + 4
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(&Ws[wb][row][col]));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(&Ws[wb][row + 4][col]));
          afr[tn] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
          afr[tn] = *reinterpret_cast<const bf16x8*>(&Ws[wb][wn0 + tn * 32 + (lane & 31)][kk * 16 + 8 * (lane >> 5)]);
        }
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          acc[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[tn], bfr[tm], acc[tn][tm], 0, 0, 0);
    }
  };

  lds_barrier();   // step 0's loads have landed
  lds_barrier();   // phase 0: step 0's W tile is built
  // phase s + 1 computes step s; six steps per iteration cover every (stage, buffer) pair
  const std::integral_constant<int, 0> c0{};
  const std::integral_constant<int, 1> c1{};
  const std::integral_constant<int, 2> c2{};
  int s = 0;
  for (; s + 6 <= steps; s += 6) {
    compute(c0, c0); lds_barrier();
    compute(c1, c1); lds_barrier();
    compute(c2, c0); lds_barrier();
    compute(c0, c1); lds_barrier();
    compute(c1, c0); lds_barrier();
    compute(c2, c1); lds_barrier();
  }
  if (s < steps) { compute(c0, c0); lds_barrier(); }
  if (s + 1 < steps) { compute(c1, c1); lds_barrier(); }
  if (s + 2 < steps) { compute(c2, c0); lds_barrier(); }
  if (s + 3 < steps) { compute(c0, c1); lds_barrier(); }
  if (s + 4 < steps) { compute(c1, c0); lds_barrier(); }

  // ---------------------------------------------------------------- epilogue
  if (nsplit > 1) {
    // fp32 partial sums of this contraction range, straight from the accumulators (lane: one row,
    // four consecutive columns per group of four registers): [range][M][Nout] for a uniform split,
    // [range][tail tile][BM][kBN] for a tail piece
    const bool tail = g.tail_tiles > 0;
    float* pp = tail ? g.part + ((int64_t)split * g.tail_tiles + tail_r) * (BM * kBN)
                     : g.part + (int64_t)split * g.M * Nout;
    const int64_t pitch = tail ? kBN : Nout;
    const int64_t r0 = tail ? m0 : 0, c0 = tail ? col0 : 0;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const f32x16& a = acc[tn][tm];
        const int64_t m = m0 + wm0 + tm * 32 + (lane & 31);
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int64_t n = col0 + wn0 + tn * 32 + 8 * rq + 4 * (lane >> 5);
          if (m < g.M && n < Nout)
            *reinterpret_cast<f32x4*>(pp + (m - r0) * pitch + (n - c0)) =
                f32x4{a[4 * rq], a[4 * rq + 1], a[4 * rq + 2], a[4 * rq + 3]};
        }
      }
    return;
  }
  // Every wave has passed the barrier after the last step, so the activation stages are free: wave
  // cw stages its WM x WN sub-tile as bf16 rows of WN values (16-byte slot c of row q at
  // c ^ ((q >> 1) & (C16 - 1))), then each store instruction writes 16 bytes per lane and whole
  // rows of the sub-tile (128 bytes when WN = 64) from consecutive lanes.
  constexpr int SUB = CW::WM * CW::WN;
  static_assert(8 * SUB <= kXStages * XSTAGE, "sub-tiles fit in the activation stages");
  constexpr int C16 = CW::WN / 8;           // 16-byte slots per row
  constexpr int RPI = 64 / C16;             // rows per store instruction
  uint16_t* stg = Xs + cw * SUB;
  auto slot = [&](int q, int c16) { return q * CW::WN + ((c16 ^ ((q >> 1) & (C16 - 1))) * 8); };
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const f32x16& a = acc[tn][tm];
      const int q = tm * 32 + (lane & 31);
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)   // columns tn * 32 + 8 rq + 4 (lane / 32) .. +3
        *reinterpret_cast<u32x2*>(stg + slot(q, 4 * tn + rq) + 4 * (lane >> 5)) =
            u32x2{pack_bf16x2(a[4 * rq], a[4 * rq + 1]), pack_bf16x2(a[4 * rq + 2], a[4 * rq + 3])};
    }
#pragma unroll
  for (int j = 0; j < CW::WM / RPI; ++j) {
    const int q = j * RPI + lane / C16, c16 = lane % C16;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + slot(q, c16));
    const int64_t m = m0 + wm0 + q, n = col0 + wn0 + 8 * c16;
    if (m < g.M && n < Nout) *reinterpret_cast<u32x4*>(g.out + m * Nout + n) = v;
  }
}

// Sum of the contraction ranges' partial sums, in range order, rounded to bf16.
__global__ __launch_bounds__(256) void gemm_ksum_kernel(const f32x4* __restrict__ part, int64_t n4, int ksplit,
                                                        u32x2* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  f32x4 a = part[i];
  for (int s = 1; s < ksplit; ++s) {
    const f32x4 b = part[(int64_t)s * n4 + i];
    a = f32x4{a[0] + b[0], a[1] + b[1], a[2] + b[2], a[3] + b[3]};
  }
  out[i] = u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
}

// Sum of the tail pieces' partial sums (tile-major: [range][tail tile][bm][kBN]), in range order,
// rounded to bf16. Workgroup w takes 32 rows of tail tile w / (bm / 32) (tile first + that); a
// thread 4 groups of 4 values, all loads of all ranges in flight together. Rows past M and columns
// past Nout were never written and are skipped.
constexpr int kKsumRows = 32;
template <int NS, bool DX>
__global__ __launch_bounds__(256) void gemm_ksum_tail_kernel(const f32x4* __restrict__ part, const GemmArgs ga,
                                                             int tail, int first, int gx, int bm) {
  const int per_tile = bm / kKsumRows;
  const int tr = blockIdx.x / per_tile, rs = blockIdx.x % per_tile, tile = first + tr;
  const int64_t m0 = (int64_t)(tile / gx) * bm + rs * kKsumRows;
  int64_t c0 = (int64_t)(tile % gx) * kBN;
  GemmArgs g = ga;
  if (!DX && ga.nw > 1) select_weight(g, ga, tile % gx, c0);
  const int64_t M = g.M, Nout = DX ? g.K : g.N;
  u32x2* __restrict__ out = reinterpret_cast<u32x2*>(g.out);
  const int per = bm * kBN / 4;   // 4-value groups per tile
  const f32x4* src = part + (int64_t)tr * per + rs * kKsumRows * (kBN / 4);
  f32x4 v[NS][4];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) v[s][i] = src[(int64_t)s * tail * per + threadIdx.x + 256 * i];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = threadIdx.x + 256 * i;
    const int64_t m = m0 + e / (kBN / 4), n = c0 + 4 * (e % (kBN / 4));
    f32x4 a = v[0][i];
#pragma unroll
    for (int s = 1; s < NS; ++s) a = f32x4{a[0] + v[s][i][0], a[1] + v[s][i][1], a[2] + v[s][i][2], a[3] + v[s][i][3]};
    if (m < M && n < Nout) out[(m * Nout + n) / 4] = u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
  }
}

// A launch plan of the fused GEMM (it depends on the shapes only, so the workspace size and the
// launch always agree): the tile height, contraction ranges of every tile (uniform split), and the
// tail. With one workgroup per CU, T tiles take ceil(T / 256) rounds of the 256 CUs; past the last
// whole round the other R = T mod 256 tiles would leave 256 - R CUs idle for a whole tile's time.
// Tail mode cuts each of those R tiles into s = 2..4 contraction ranges (at least 8 steps each),
// so the last round holds R s shorter pieces; gemm_ksum_tail_kernel then adds them. The forward:
//   * 256-row tiles when there are at least 192 of them (then the tail, when R <= 128);
//   * else, above 128 tokens, 256-row tiles with the contraction cut into ks = 2..4 ranges (at
//     least 8 steps each) when that makes at least 192 workgroups: a dequantised W tile then
//     feeds 256 token rows instead of 128, which halves the dequantisation per flop (the k and v
//     projections of a layer: 1024 output columns);
//   * else 128-row tiles (64 at most 64 tokens), with the contraction cut into up to 4 (8 for
//     64-row tiles) ranges, as many as keep the workgroups within one round (few_tile_ranges).
// The dX GEMM takes 256-row tiles when there are at least 192 of them (with the tail), else 128 or
// 64 with the contraction cut the same way: at 16 tokens a 4096x4096 weight makes 32 tiles, and a
// tile's time follows its steps.
struct GemmPlan {
  int bm, ks;
  int whole, tail, tsplit;   // tail mode when tail > 0
};

static void plan_tail(GemmPlan& p, int64_t tiles, int64_t steps) {
  const int64_t R = tiles % 256;
  if (tiles <= 256 || R == 0) return;
  const int64_t s = min((int64_t)4, min(256 / R, steps / 8));
  if (s < 2 || (tiles - R) % 8 || (R * s) % 8) return;   // each XCD takes an equal share of both
  p.whole = (int)(tiles - R);
  p.tail = (int)R;
  p.tsplit = (int)s;
}

// Contraction ranges of 128- and 64-row tiles: as many as keep the workgroups within one round of
// the 256 CUs, at most 4 (8 for 64-row tiles), each of at least 8 steps (two ranges from 8 steps
// on). The last range then always keeps a step: ks <= 8 and ks <= steps / 8 give (ks - 1) *
// ceil(steps / ks) < steps.
static int few_tile_ranges(int64_t tiles, int64_t steps, int bm) {
  if (steps < 8) return 1;
  const int64_t by_steps = steps / 8 > 2 ? steps / 8 : 2;
  const int64_t ks = min((int64_t)(bm == 64 ? 8 : 4), min(by_steps, 256 / tiles));
  return ks > 1 ? (int)ks : 1;
}

static GemmPlan fwd_gemm_plan(int64_t M, int64_t N, int64_t K) {
  GemmPlan p{0, 1, 0, 0, 0};
  const int64_t gx = (N + kBN - 1) / kBN, steps = (K + kBK - 1) / kBK;
  const int64_t t256 = gx * ((M + 255) / 256);
  if (M > 128 && t256 >= 192) {
    p.bm = 256;
    plan_tail(p, t256, steps);
    return p;
  }
  if (M > 128) {
    const int64_t ks = min((int64_t)4, min(steps / 8, (256 + t256 - 1) / t256));
    if (ks > 1 && t256 * ks >= 192) {
      p.bm = 256;
      p.ks = (int)ks;
      return p;
    }
  }
  p.bm = M <= 64 ? 64 : 128;
  p.ks = few_tile_ranges(gx * ((M + p.bm - 1) / p.bm), steps, p.bm);
  return p;
}

static GemmPlan dx_gemm_plan(int64_t M, int64_t N, int64_t K) {
  GemmPlan p{0, 1, 0, 0, 0};
  const int64_t gx = (K + kBN - 1) / kBN, steps = (N + kBK - 1) / kBK;
  const int64_t t256 = gx * ((M + 255) / 256);
  p.bm = (M > 128 && t256 >= 192) ? 256 : M > 64 ? 128 : 64;
  if (p.bm == 256) {
    plan_tail(p, t256, steps);
    return p;
  }
  p.ks = few_tile_ranges(gx * ((M + p.bm - 1) / p.bm), steps, p.bm);
  return p;
}

static size_t plan_part_floats(const GemmPlan& p, int64_t M, int64_t Nout) {
  if (p.ks > 1) return (size_t)p.ks * (size_t)M * (size_t)Nout;
  if (p.tail > 0) return (size_t)p.tsplit * (size_t)p.tail * (size_t)p.bm * kBN;
  return 0;
}

size_t fwd_gemm_part_floats(int64_t M, int64_t N, int64_t K) { return plan_part_floats(fwd_gemm_plan(M, N, K), M, N); }
size_t dx_gemm_part_floats(int64_t M, int64_t N, int64_t K) { return plan_part_floats(dx_gemm_plan(M, N, K), M, K); }

template <bool DX, bool F32S>
static hipError_t launch_gemm_t(GemmArgs g, const GemmPlan& p, hipStream_t stream) {
  const int64_t Nout = DX ? g.K : g.N;
  const int gx = g.nw > 1 ? g.gx_total : (int)((Nout + kBN - 1) / kBN);
  const int gy = (int)((g.M + p.bm - 1) / p.bm);
  g.ksplit = p.ks;
  g.whole_tiles = p.whole;
  g.tail_tiles = p.tail;
  g.tail_split = p.tsplit;
  const dim3 grid = p.tail > 0 ? dim3((unsigned)(p.whole + p.tail * p.tsplit)) : dim3(gx, gy * p.ks);
  if (p.bm == 256) hipLaunchKernelGGL((qlora_gemm_kernel<DX, 256, F32S>), grid, dim3(kThreads), 0, stream, g);
  else if (p.bm == 128) hipLaunchKernelGGL((qlora_gemm_kernel<DX, 128, F32S>), grid, dim3(kThreads), 0, stream, g);
  else hipLaunchKernelGGL((qlora_gemm_kernel<DX, 64, F32S>), grid, dim3(kThreads), 0, stream, g);
  if (p.ks > 1) {
    const int64_t n4 = g.M * Nout / 4;
    hipLaunchKernelGGL(gemm_ksum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                       (const f32x4*)g.part, n4, p.ks, reinterpret_cast<u32x2*>(g.out));
  } else if (p.tail > 0) {
    const dim3 kg((unsigned)(p.tail * (p.bm / kKsumRows)));
    const f32x4* src = (const f32x4*)g.part;
    if (p.tsplit == 2) hipLaunchKernelGGL((gemm_ksum_tail_kernel<2, DX>), kg, dim3(256), 0, stream, src, g, p.tail, p.whole, gx, p.bm);
    else if (p.tsplit == 3) hipLaunchKernelGGL((gemm_ksum_tail_kernel<3, DX>), kg, dim3(256), 0, stream, src, g, p.tail, p.whole, gx, p.bm);
    else hipLaunchKernelGGL((gemm_ksum_tail_kernel<4, DX>), kg, dim3(256), 0, stream, src, g, p.tail, p.whole, gx, p.bm);
  }
  return hipGetLastError();
}

// Without room for partial sums (part null): one contraction range for every tile.
static void plan_without_part(GemmPlan& p) {
  p.ks = 1;
  p.whole = p.tail = p.tsplit = 0;
}

hipError_t launch_fwd_gemm(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                           const float* absmax, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                           const float* u, const uint16_t* B, int r, float scale, uint16_t* y,
                           float* part, int book, hipStream_t stream) {
  GemmPlan p = fwd_gemm_plan(M, N, K);
  if (!part) {   // at the tile height the plan takes without splitting
    plan_without_part(p);
    const int64_t gx = (N + kBN - 1) / kBN;
    p.bm = (M > 128 && gx * ((M + 255) / 256) >= 192) ? 256 : M > 64 ? 128 : 64;
  }
  GemmArgs g{packed, scale_q, scale_c2, absmax, N, K, x, M, u, B, r, scale, y, 1, part, 0, 0, 0, {}};
  if (!codes_of(book, g.codes)) return hipErrorInvalidValue;
  return absmax ? launch_gemm_t<false, true>(g, p, stream) : launch_gemm_t<false, false>(g, p, stream);
}

hipError_t launch_dx_gemm(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                          const float* absmax, int64_t N, int64_t K, const uint16_t* dy, int64_t M,
                          const float* v, const uint16_t* A, int r, float scale, uint16_t* dx,
                          float* part, int book, hipStream_t stream) {
  GemmPlan p = dx_gemm_plan(M, N, K);
  if (!part) plan_without_part(p);
  GemmArgs g{packed, scale_q, scale_c2, absmax, N, K, dy, M, v, A, r, scale, dx, 1, part, 0, 0, 0, {}};
  if (!codes_of(book, g.codes)) return hipErrorInvalidValue;
  return absmax ? launch_gemm_t<true, true>(g, p, stream) : launch_gemm_t<true, false>(g, p, stream);
}

// The grouped forward (forward only, 256-row tiles): its column tiles run over the weights in
// turn, and the tail is planned over all of them. Not eligible (false) when the group's tiles would
// not take 256-row tiles by themselves; the caller then launches the linears one by one.
static bool fwd_group_plan(int count, const int64_t* N, int64_t M, int64_t K, GemmPlan& p, int& gx_total) {
  gx_total = 0;
  for (int i = 0; i < count; ++i) gx_total += (int)((N[i] + kBN - 1) / kBN);
  const int64_t t256 = (int64_t)gx_total * ((M + 255) / 256), steps = (K + kBK - 1) / kBK;
  p = GemmPlan{256, 1, 0, 0, 0};
  if (count < 2 || count > kMaxGroup || M <= 128 || t256 < 192) return false;
  plan_tail(p, t256, steps);
  return true;
}

bool fwd_group_eligible(int count, const int64_t* N, int64_t M, int64_t K) {
  GemmPlan p;
  int gx;
  return fwd_group_plan(count, N, M, K, p, gx);
}

size_t fwd_group_part_floats(int count, const int64_t* N, int64_t M, int64_t K) {
  GemmPlan p;
  int gx;
  if (!fwd_group_plan(count, N, M, K, p, gx)) return 0;
  return plan_part_floats(p, M, 0);
}

hipError_t launch_fwd_gemm_group(int count, const FwdGroupItem* it, int64_t K, const uint16_t* x, int64_t M,
                                 int r, float scale, float* part, int book, hipStream_t stream) {
  int64_t N[kMaxGroup];
  for (int i = 0; i < count && i < kMaxGroup; ++i) N[i] = it[i].N;
  GemmPlan p;
  int gx_total;
  if (!fwd_group_plan(count, N, M, K, p, gx_total)) return hipErrorInvalidValue;
  if (!part) plan_without_part(p);
  const bool f32s = it[0].absmax != nullptr;
  GemmArgs g{it[0].packed, it[0].scale_q, it[0].scale_c2, it[0].absmax, it[0].N, K, x, M, it[0].u, it[0].B, r, scale,
             it[0].y, 1, part, 0, 0, 0, {}, count, gx_total, {}};
  if (!codes_of(book, g.codes)) return hipErrorInvalidValue;
  int tile0 = 0;
  for (int i = 0; i < count; ++i) {
    if ((it[i].absmax != nullptr) != f32s) return hipErrorInvalidValue;
    g.w[i] = GemmWeight{it[i].packed, it[i].scale_q, it[i].scale_c2, it[i].absmax, it[i].N, nullptr, it[i].u, it[i].B,
                        it[i].y, tile0};
    tile0 += (int)((it[i].N + kBN - 1) / kBN);
  }
  return f32s ? launch_gemm_t<false, true>(g, p, stream) : launch_gemm_t<false, false>(g, p, stream);
}

// The grouped dX (256-row tiles, no split): every weight's M x K tiles in turn, each linear with its
// own dY, v, A and dX. Eligible when M > 128 and the tiles of all weights number at least 192.
bool dx_group_eligible(int count, int64_t M, int64_t K) {
  const int64_t t = ((K + kBN - 1) / kBN) * ((M + 255) / 256);
  return count >= 2 && count <= kMaxGroup && M > 128 && t * count >= 192;
}

hipError_t launch_dx_gemm_group(int count, const DxGroupItem* it, int64_t K, int64_t M, int r, float scale,
                                int book, hipStream_t stream) {
  if (!dx_group_eligible(count, M, K)) return hipErrorInvalidValue;
  const bool f32s = it[0].absmax != nullptr;
  GemmArgs g{it[0].packed, it[0].scale_q, it[0].scale_c2, it[0].absmax, it[0].N, K, it[0].dy, M, it[0].v, it[0].A, r,
             scale, it[0].dx, 1, nullptr, 0, 0, 0, {}, count, 0, {}};
  if (!codes_of(book, g.codes)) return hipErrorInvalidValue;
  for (int i = 0; i < count; ++i) {
    if ((it[i].absmax != nullptr) != f32s) return hipErrorInvalidValue;
    g.w[i] = GemmWeight{it[i].packed, it[i].scale_q, it[i].scale_c2, it[i].absmax, it[i].N, it[i].dy, it[i].v, it[i].A,
                        it[i].dx, 0};
  }
  const int gx = (int)((K + kBN - 1) / kBN), gy = (int)((M + 255) / 256);
  const dim3 grid((unsigned)(gx * gy * count));
  if (f32s) hipLaunchKernelGGL((qlora_gemm_kernel<true, 256, true>), grid, dim3(kThreads), 0, stream, g);
  else hipLaunchKernelGGL((qlora_gemm_kernel<true, 256, false>), grid, dim3(kThreads), 0, stream, g);
  return hipGetLastError();
}

}  // namespace nf4
