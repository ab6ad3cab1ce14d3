// Adapter (LoRA) kernels of the adapted linear (gfx950).
//
// "QLoRA, explained", The forward pass and gradients: the adapter gradients are LoRA's with the
// dequantised weight in place of the original, dB = s G A^T and dA = s B^T G with G = dY^T X.
// Computed here without forming G (N x K):
//   u  = X A^T   [M x r]   (forward; saved for the backward)
//   v  = dY B    [M x r]   (backward)
//   dA = s v^T X [r x K]   and   dB = s dY^T u [N x r]     (fp32, optionally accumulated)
//
// All four are passes over one bf16 matrix Q [M x C] (X or dY) that the pass reads once:
//   down:  Dn[m][j] = sum_c Q[m][c] R(c, j)    R(c, j) = A[j][c] (A is r x C) or B[c][j] (B is C x r)
//   grad:  Gr[c][j] = sum_m Q[m][c] P[m][j]    P = u or v, fp32, as a bf16 hi + lo pair
// The backward's pass over dY does both at once (v and dB), so dY is read once for the adapter.
// A workgroup takes 256 (or, above rank 64, 128) rows and a range of columns, streaming 64-column
// steps of Q through LDS with LDS-DMA loads; the down products accumulate over its columns, the
// grad products of each step are complete for its rows. Partial results go to a workspace and
// lora_reduce_kernel sums them in a fixed order, so results are bitwise reproducible.
#include "common.h"
#include "launch.h"

namespace nf4 {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
constexpr int kStepC = 64;                     // Q columns per step

// 16-lane transpose read of an LDS tile stored [contraction][column] with pitch `pitch`:
// returns, for lane (j = lane % 16, grp = lane / 16), the 8 contraction values
// rows 8*grp .. 8*grp+7 of column col0 + j, as an MFMA operand fragment.
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* tile, int pitch, int col0, int lane) {
  const int j = lane & 15, grp = lane >> 4;
  const uint16_t* p = tile + (8 * grp + (j >> 2)) * pitch + col0 + 4 * (j & 3);
  bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
  bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 4 * pitch));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Q tiles in LDS: rows of 64 bf16 (128 bytes); the 16-byte chunk c of row m sits at slot
// c ^ ((m >> 1) & 7), so 16-lane groups reading one chunk of 16 consecutive rows hit distinct banks.
__device__ __forceinline__ int q_elem(int m, int c) {
  return m * kStepC + ((((c >> 3) ^ ((m >> 1) & 7)) << 3) | (c & 7));
}

// transpose read of the swizzled Q tile: lane (j, grp) receives rows m0 + 8*grp .. +7 of column
// c0 + j (c0 a multiple of 16)
__device__ __forceinline__ bf16x8 q_tr_frag(const uint16_t* tile, int m0, int c0, int lane) {
  const int j = lane & 15, grp = lane >> 4;
  const int m = m0 + 8 * grp + (j >> 2), c = c0 + 4 * (j & 3);
  bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tile + q_elem(m, c)));
  bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tile + q_elem(m + 4, c)));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

struct LoraPassArgs {
  const uint16_t* Q;        // [M x C] bf16
  int64_t M, C;
  const uint16_t* R;        // down operand: A [r x C] (RT = false) or B [C x r] (RT = true)
  // grad operand [M x r] fp32: the r / rl operands P[i], each [M x rl], side by side (linears of rank rl
  // that share Q; one operand, rl = r, otherwise)
  const float* P[4];
  int rl;
  int r;
  int64_t crange;           // columns per workgroup column range (a multiple of kStepC)
  float* part_down;         // [column ranges][M][r]
  float* part_grad;         // [r / rl][row blocks][C][rl]: each operand's partial sums on their own
  int mblocks;              // row blocks (workgroup b of the pass: row block b % mblocks, range b / mblocks)
};

// Passes of one kind and rank over different matrices, as one launch: workgroups [first[k],
// first[k + 1]) run pass k. Each pass computes what it computes alone.
constexpr int kMaxPassGroup = 4;
struct LoraPassGroup {
  LoraPassArgs a[kMaxPassGroup];
  int first[kMaxPassGroup];
  int n;
};

// RMAX: the rank rounded up to 16, 32, 64 or 128 (the tiles are sized for it); QS: Q stages in
// LDS (QS - 1 steps in flight). With RMAX = 16 the grad operand fragments stay in registers.
template <int MB, int RMAX, int QS, bool DOWN, bool GRAD, bool RT>
__global__ __launch_bounds__(256) void lora_pass_kernel(const LoraPassGroup pg) {
  // this workgroup's pass, chosen by scalar selects (no indexing of the argument block)
  LoraPassArgs a = pg.a[0];
  int b0 = 0;
#pragma unroll
  for (int k = 1; k < kMaxPassGroup; ++k)
    if (k < pg.n && (int)blockIdx.x >= pg.first[k]) {
      a = pg.a[k];
      b0 = pg.first[k];
    }
  const int mbi = ((int)blockIdx.x - b0) % a.mblocks, cri = ((int)blockIdx.x - b0) / a.mblocks;
  constexpr bool R16 = RMAX == 16;
  constexpr int NQ = MB / 32;                           // Q DMA loads per wave per step
  constexpr int RTILE = DOWN ? kStepC * RMAX : 8;       // R tile elements per stage
  constexpr int PP = (GRAD ? RMAX : 0) + 8;             // pitch of the P tiles
  __shared__ __attribute__((aligned(16))) uint16_t Qs[QS][MB * kStepC];
  __shared__ __attribute__((aligned(16))) uint16_t Rs[QS][RTILE];
  __shared__ __attribute__((aligned(16))) uint16_t Ph[GRAD ? MB : 1][PP];
  __shared__ __attribute__((aligned(16))) uint16_t Pl[GRAD ? MB : 1][PP];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = R16 ? 16 : a.r, RT16 = r / 16;
  const int64_t m0 = (int64_t)mbi * MB;
  const int64_t rows_valid = min(a.M - m0, (int64_t)MB);
  const int64_t c_begin = (int64_t)cri * a.crange;
  const int64_t c_end = min(a.C, c_begin + a.crange);
  const int nsteps = (int)((c_end - c_begin + kStepC - 1) / kStepC);

  // ---- DMA of one step: Q rows m0.., columns c0 .. c0+63 (swizzled), then the R tile
  constexpr int rdma = (RMAX + 31) / 32;   // R loads per wave per step (waves past the tile repeat one)
  auto issue = [&](int t) {
    const int64_t c0 = c_begin + (int64_t)t * kStepC;
    const int st = t % QS;
    const int valid_chunks = (int)min((int64_t)8, (a.C - c0 + 7) / 8);
    {
      const uint16_t* base = a.Q + m0 * a.C + c0;
      const int nrec = (int)(rows_valid * a.C * 2 - c0 * 2);
      __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nrec, kRsrcFlags);
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const int slot = (wave * NQ + j) * 64 + lane;
        const int row = slot >> 3, c = (slot & 7) ^ ((row >> 1) & 7);
        const uint32_t off = c < valid_chunks ? (uint32_t)row * (uint32_t)(a.C * 2) + (uint32_t)c * 16u : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(&Qs[st][(wave * NQ + j) * 64 * 8]), 16, off, 0, 0, 0);
      }
    }
    if (DOWN) {
      // R tile of the step: RT = false, rows j < r of A, columns c0 .. c0+63, swizzled like Q;
      // RT = true, rows c0 .. c0+63 of B (r columns each), contiguous. Either is r/8 loads of
      // 64 lanes x 16 bytes; load i goes to wave i % 4.
      for (int k = 0; k < rdma; ++k) {
        int i = wave + 4 * k;
        if (i >= r / 8) i = (r / 8) - 1 - ((i - r / 8) % (r / 8));   // repeat an existing load
        const int slot = i * 64 + lane;
        uint32_t off;
        __amdgpu_buffer_rsrc_t rs;
        if (RT) {
          rs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.R + c0 * r), (short)0,
                                                 (int)((a.C - c0) * r * 2), kRsrcFlags);
          off = (uint32_t)slot * 16u;
        } else {
          rs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.R + c0), (short)0,
                                                 (int)(r * a.C * 2 - c0 * 2), kRsrcFlags);
          const int row = slot >> 3, c = (slot & 7) ^ ((row >> 1) & 7);
          off = c < valid_chunks ? (uint32_t)row * (uint32_t)(a.C * 2) + (uint32_t)c * 16u : kOutOfRange;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(&Rs[st][i * 64 * 8]), 16, off, 0, 0, 0);
      }
    }
  };

  // ---- P rows of the block as bf16 hi + lo (grad)
  if (GRAD) {
    const int cols4 = r / 4;
    for (int q = tid; q < MB * cols4; q += 256) {
      const int row = q / cols4, c4 = (q % cols4) * 4;
      const int li = c4 / a.rl;
      const float* src = a.P[0];
      if (li == 1) src = a.P[1];
      if (li == 2) src = a.P[2];
      if (li == 3) src = a.P[3];
      f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
      if (row < rows_valid) v = *reinterpret_cast<const f32x4*>(src + (m0 + row) * a.rl + c4 - li * a.rl);
      const uint32_t h01 = pack_bf16x2(v[0], v[1]), h23 = pack_bf16x2(v[2], v[3]);
      const uint32_t l01 = pack_bf16x2(v[0] - __uint_as_float(h01 << 16), v[1] - __uint_as_float(h01 & 0xFFFF0000u));
      const uint32_t l23 = pack_bf16x2(v[2] - __uint_as_float(h23 << 16), v[3] - __uint_as_float(h23 & 0xFFFF0000u));
      *reinterpret_cast<u32x2*>(&Ph[row][c4]) = u32x2{h01, h23};
      *reinterpret_cast<u32x2*>(&Pl[row][c4]) = u32x2{l01, l23};
    }
  }

  // rank 16: every step multiplies by the same P fragments; read them once
  bf16x8 pfr[R16 && GRAD ? MB / 32 : 1][2];
  if (R16 && GRAD) {
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < MB / 32; ++kk) {
      pfr[kk][0] = tr_frag(&Ph[kk * 32][0], PP, 0, lane);
      pfr[kk][1] = tr_frag(&Pl[kk * 32][0], PP, 0, lane);
    }
  }

  // ---- accumulators. down: wave owns rows wave * MB/4 ..; grad: wave owns columns 16 wave .. of
  // each step.
  // where the 16 grad columns of tile jt go: operand jt * 16 / rl, its columns from jt * 16 % rl
  float* gdst[RMAX / 16];
#pragma unroll
  for (int jt = 0; jt < RMAX / 16; ++jt) {
    const int li = GRAD && jt < RT16 ? jt * 16 / a.rl : 0;
    gdst[jt] = a.part_grad + ((int64_t)li * a.mblocks + mbi) * a.C * a.rl + jt * 16 - li * a.rl;
  }

  constexpr int MT = MB / 64;   // 16-row tiles of a wave (down)
  f32x4 dacc[DOWN ? MT : 1][RMAX / 16];
  f32x4 gacc[RMAX / 16];
#pragma unroll
  for (int i = 0; i < (DOWN ? MT : 1); ++i)
#pragma unroll
    for (int j = 0; j < RMAX / 16; ++j) dacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int t) {
    const int st = t % QS;
    const uint16_t* qs = &Qs[st][0];
    const int64_t c0 = c_begin + (int64_t)t * kStepC;
    if (DOWN) {
      // D lane l: column m = l % 16 of the row tile, rows j = jt*16 + 4 (l / 16) .. +3
#pragma unroll
      for (int kk = 0; kk < kStepC / 32; ++kk) {
        bf16x8 bq[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = wave * (MB / 4) + mt * 16 + (lane & 15);
          bq[mt] = *reinterpret_cast<const bf16x8*>(qs + q_elem(m, kk * 32 + 8 * (lane >> 4)));
        }
#pragma unroll
        for (int jt = 0; jt < RMAX / 16; ++jt) {
          if (jt < RT16) {
            bf16x8 ar;
            if (RT) {
              ar = tr_frag(&Rs[st][kk * 32 * r], r, jt * 16, lane);
            } else {
              const int j = jt * 16 + (lane & 15);
              ar = *reinterpret_cast<const bf16x8*>(&Rs[st][q_elem(j, kk * 32 + 8 * (lane >> 4))]);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              dacc[mt][jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar, bq[mt], dacc[mt][jt], 0, 0, 0);
          }
        }
      }
    }
    if (GRAD) {
      // D lane l: column c = 16 wave + l % 16 of the step, rows j = jt*16 + 4 (l / 16) .. +3
#pragma unroll
      for (int j = 0; j < RMAX / 16; ++j) gacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < MB / 32; ++kk) {
        const bf16x8 bq = q_tr_frag(qs, kk * 32, wave * 16, lane);
        if (R16) {
          gacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pfr[kk][0], bq, gacc[0], 0, 0, 0);
          gacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pfr[kk][1], bq, gacc[0], 0, 0, 0);
        } else {
#pragma unroll
          for (int jt = 0; jt < RMAX / 16; ++jt) {
            if (jt < RT16) {
              const bf16x8 ph = tr_frag(&Ph[kk * 32][0], PP, jt * 16, lane);
              const bf16x8 pl = tr_frag(&Pl[kk * 32][0], PP, jt * 16, lane);
              gacc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, bq, gacc[jt], 0, 0, 0);
              gacc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, bq, gacc[jt], 0, 0, 0);
            }
          }
        }
      }
      const int64_t c = c0 + wave * 16 + (lane & 15);
      if (c < a.C) {
#pragma unroll
        for (int jt = 0; jt < RMAX / 16; ++jt)
          if (jt < RT16) *reinterpret_cast<f32x4*>(gdst[jt] + c * a.rl + 4 * (lane >> 4)) = gacc[jt];
      }
    }
  };

  // ---- pipeline: QS-1 steps in flight. Step t: start the DMA of step t+QS-1, wait until step
  // t's loads have landed (later steps' loads may stay in flight: vector-memory loads complete in
  // issue order), barrier, compute, barrier (the stage is refilled next).
  constexpr int PER = NQ + (DOWN ? rdma : 0);          // loads per wave per step
  static_assert((QS - 1) * PER <= 63, "vmcnt range");
  for (int t = 0; t < QS - 1 && t < nsteps; ++t) issue(t);
  for (int t = 0; t < nsteps; ++t) {
    if (t + QS - 1 < nsteps) {
      issue(t + QS - 1);
      wait_vmcnt<(QS - 1) * PER>();   // the loads of steps t+1 .. t+QS-1 may stay in flight
    } else {
      // no more issues: steps t+1 .. nsteps-1 may stay in flight
      const int ahead = nsteps - 1 - t;
      if (QS > 5 && ahead >= 4) wait_vmcnt<(QS > 5 ? 4 : 0) * PER>();
      else if (QS > 4 && ahead >= 3) wait_vmcnt<(QS > 4 ? 3 : 0) * PER>();
      else if (QS > 3 && ahead >= 2) wait_vmcnt<(QS > 3 ? 2 : 0) * PER>();
      else if (QS > 2 && ahead >= 1) wait_vmcnt<(QS > 2 ? 1 : 0) * PER>();
      else wait_vmcnt<0>();
    }
    lds_barrier();
    compute(t);
    lds_barrier();
  }

  if (DOWN) {
    float* dst = a.part_down + (int64_t)cri * a.M * r;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int64_t m = m0 + wave * (MB / 4) + mt * 16 + (lane & 15);
      if (m < a.M) {
#pragma unroll
        for (int jt = 0; jt < RMAX / 16; ++jt)
          if (jt < RT16) *reinterpret_cast<f32x4*>(dst + m * r + jt * 16 + 4 * (lane >> 4)) = dacc[mt][jt];
      }
    }
  }
}

// Ordered sums of partial results. A job: out[i] = scale * (sum over p < nparts, in order, of
// part[p * count + i]) (+ out[i]); with `transpose`, part is [C][r] and out is [r][C]. One launch
// serves up to kMaxReduceJobs jobs (blocks [first[k], first[k + 1]) take job k). A thread takes one
// element of the partials' own order (so the loads of a wave are contiguous; a transposed job
// scatters only its one store) and issues the loads of 8 partials at a time before adding them in
// order; the sums are latency-bound chains, so one output per thread gives the most chains in flight.
struct ReduceJob {
  const float* part;
  int nparts;
  int64_t count, C;
  int r, transpose, accumulate;
  float scale;
  float* out;
};
constexpr int kMaxReduceJobs = 8;
struct ReduceJobs {
  ReduceJob j[kMaxReduceJobs];
  int first[kMaxReduceJobs];
  int n;
};

__global__ __launch_bounds__(256) void lora_reduce_kernel(const ReduceJobs js) {
  // the job of this workgroup, chosen by scalar selects (no indexing of the argument block)
  ReduceJob jb = js.j[0];
  int b0 = 0;
#pragma unroll
  for (int k = 1; k < kMaxReduceJobs; ++k)
    if (k < js.n && (int)blockIdx.x >= js.first[k]) {
      jb = js.j[k];
      b0 = js.first[k];
    }
  const int64_t src = (int64_t)((int)blockIdx.x - b0) * 256 + threadIdx.x;
  if (src >= jb.count) return;
  // part [C][r] -> out [r][C]: element (c, j) = src goes to j * C + c
  const int64_t i = jb.transpose ? (src % jb.r) * jb.C + src / jb.r : src;
  float s = 0.f;
  for (int p0 = 0; p0 < jb.nparts; p0 += 8) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = jb.part[(int64_t)min(p0 + q, jb.nparts - 1) * jb.count + src];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (p0 + q < jb.nparts) s += v[q];
  }
  const float x = s * jb.scale;
  jb.out[i] = jb.accumulate ? jb.out[i] + x : x;
}

// ------------------------------------------------------------------------------------------
// Work split of a pass: row blocks of 256 rows (128 above rank 64) and column ranges of whole steps,
// about 256 workgroups in all with at least 4 steps per workgroup where the matrix allows it. The
// grad partial sums (one [C][r] array per row block) cost as many bytes as Q itself at M = 4096,
// r = 64 with 128-row blocks; 256-row blocks halve them.
static int pass_rmax(int r) { return r <= 16 ? 16 : r <= 32 ? 32 : r <= 64 ? 64 : 128; }

LoraPassPlan lora_pass_plan(int64_t M, int64_t C, int r) {
  LoraPassPlan p;
  p.mb = pass_rmax(r) == 128 ? 128 : 256;
  p.mblocks = (int)((M + p.mb - 1) / p.mb);
  const int64_t steps = (C + kStepC - 1) / kStepC;
  int64_t want = (256 + p.mblocks - 1) / p.mblocks;
  if (want > (steps + 3) / 4) want = (steps + 3) / 4;
  if (want < 1) want = 1;
  const int64_t steps_per = (steps + want - 1) / want;
  p.crange = steps_per * kStepC;
  p.cranges = (int)((C + p.crange - 1) / p.crange);
  return p;
}

size_t lora_pass_ws_floats(int64_t M, int64_t C, int r, bool down, bool grad) {
  const LoraPassPlan p = lora_pass_plan(M, C, r);
  return (down ? (size_t)p.cranges * M * r : 0) + (grad ? (size_t)p.mblocks * C * r : 0);
}

// Q stages that fit one workgroup's LDS (one workgroup per CU), at most 6: 3 at ranks up to 32, 2
// above
template <int MB, int RMAX, bool DOWN, bool GRAD>
constexpr int pass_stages() {
  constexpr int stage = MB * kStepC * 2 + (DOWN ? kStepC * RMAX * 2 : 16);
  constexpr int pbytes = GRAD ? 2 * MB * (RMAX + 8) * 2 : 2 * 16;
  constexpr int q = (163840 - pbytes - 512) / stage;
  return q > 6 ? 6 : q;
}

template <int MB, int RMAX, bool DOWN, bool GRAD, bool RT>
static void launch_pass_t(unsigned blocks, const LoraPassGroup& pg, hipStream_t stream) {
  constexpr int QS = pass_stages<MB, RMAX, DOWN, GRAD>();
  static_assert(QS >= 2, "two stages at least");
  hipLaunchKernelGGL((lora_pass_kernel<MB, RMAX, QS, DOWN, GRAD, RT>), dim3(blocks), dim3(256), 0, stream, pg);
}

// n passes of one rank (each with its plan p[k]) as one launch
template <bool DOWN, bool GRAD, bool RT>
static void launch_passes(int n, const LoraPassPlan* p, const LoraPassArgs* a, hipStream_t stream) {
  LoraPassGroup pg{};
  unsigned blocks = 0;
  for (int k = 0; k < n; ++k) {
    pg.a[k] = a[k];
    pg.a[k].mblocks = p[k].mblocks;
    pg.first[k] = (int)blocks;
    blocks += (unsigned)p[k].mblocks * (unsigned)p[k].cranges;
  }
  pg.n = n;
  switch (pass_rmax(a[0].r)) {
    case 16: launch_pass_t<256, 16, DOWN, GRAD, RT>(blocks, pg, stream); break;
    case 32: launch_pass_t<256, 32, DOWN, GRAD, RT>(blocks, pg, stream); break;
    case 64: launch_pass_t<256, 64, DOWN, GRAD, RT>(blocks, pg, stream); break;
    default: launch_pass_t<128, 128, DOWN, GRAD, RT>(blocks, pg, stream); break;
  }
}

template <bool DOWN, bool GRAD, bool RT>
static void launch_pass(const LoraPassPlan& p, const LoraPassArgs& a, hipStream_t stream) {
  launch_passes<DOWN, GRAD, RT>(1, &p, &a, stream);
}

static ReduceJob reduce_job(const float* part, int nparts, int64_t count, int64_t C, int r, bool transpose,
                            float scale, int accumulate, float* out) {
  return ReduceJob{part, nparts, count, C, r, transpose ? 1 : 0, accumulate, scale, out};
}

static void launch_reduce(const ReduceJob* jobs, int n, hipStream_t stream) {
  ReduceJobs js{};
  int blocks = 0;
  for (int k = 0; k < n; ++k) {
    js.j[k] = jobs[k];
    js.first[k] = blocks;
    blocks += (int)((jobs[k].count + 255) / 256);
  }
  js.n = n;
  hipLaunchKernelGGL(lora_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, js);
}

// ------------------------------------------------------------------------------------------
// u = X A^T at rank 16 in one launch, without partial sums in memory (its contraction runs over K only, so
// a workgroup can own whole rows): a workgroup owns 16 rows of X and all of K. Its 16 waves take
// groups of 8 adjacent 32-column chunks in turn (wave w: chunks 8 w .. 8 w + 7, then those 128
// chunks on), in batches of NB chunks (NB divides 8). A wave adds its chunks in the same order
// whatever NB is, so u comes out bit for bit the same for any number of tiles in the launch.
// The MFMA operand layout (lane (row = lane % 16, g = lane / 16): columns 8 g .. 8 g + 7 of the
// chunk in its row) would have each load instruction touch 16 rows at 64 bytes each; instead a wave
// loads each batch of X and of every tile of A row by row, 64 NB contiguous bytes a row (whole
// 128-byte lines from NB = 2 on) with consecutive lanes on consecutive 16-byte pieces, stores it to
// its own LDS slice (pieces XOR-swizzled by row against bank conflicts) and reads it back in the
// operand layout; v_mfma_f32_16x16x32_bf16 then accumulates u[row][16 t + j]. The workgroup sums
// the 16 waves in LDS in wave order at the end.
constexpr int kUWaves = 16;
constexpr int kUGroup = 8;   // adjacent chunks per wave before the next wave's

// The 16-row tiles of A that one launch multiplies x by, and where each tile's 16 columns of u go:
// tile t reads rows A[t] .. +15 (row pitch K) and writes u[t][m * ustride + 0..15]. One linear of
// rank r has r / 16 consecutive tiles; the linears of a group at rank 16 have one tile each.
struct UTiles {
  const uint16_t* A[8];
  float* u[8];
  int ustride;
};

// chunks per batch: the wave's LDS slice, (1 + NT) NB KB, stays at 9 KB or less
template <int NT>
constexpr int u_batch() { return NT == 1 ? 4 : NT <= 3 ? 2 : 1; }

template <int NT>   // tiles
__global__ __launch_bounds__(kUWaves * 64) void lora_u_kernel(const uint16_t* __restrict__ X, int64_t M,
                                                            int64_t K, const UTiles ut) {
  constexpr int NB = u_batch<NT>();
  constexpr int P = 4 * NB;            // 16-byte pieces of a row in a batch
  constexpr int RI = 64 / P;           // rows per load instruction
  constexpr int SLICE = (1 + NT) * 16 * P;   // pieces in a wave's slice
  constexpr int r = 16 * NT;
  constexpr int STAGE = kUWaves * SLICE, RED = kUWaves * NT * 64;
  __shared__ u32x4 lds[STAGE > RED ? STAGE : RED];
  static_assert(kUGroup % NB == 0, "a batch stays inside one group of chunks");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  const int64_t nchunks = K / 32;
  u32x4* slice = lds + wave * SLICE;
  // slot of piece p of row m of matrix q (0: X, 1 + t: tile t of A) in the slice
  auto slot = [&](int q, int m, int p) {
    const int sw = P >= 8 ? (m & 7) : ((m >> 1) & 3);
    return (q * 16 + m) * P + (p ^ sw);
  };
  // the loads: instruction i of a matrix covers rows RI i + lane / P, piece lane % P
  const int lp = lane % P;
  const uint16_t* xsrc[16 / RI];
#pragma unroll
  for (int i = 0; i < 16 / RI; ++i) xsrc[i] = X + min(m0 + RI * i + lane / P, M - 1) * K + 8 * (lp & 3);
  const int64_t aoff = (int64_t)(lane / P) * K + 8 * (lp & 3);

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t k0 = 0;; k0 += NB) {
    const int64_t c0 = ((k0 / kUGroup) * kUWaves + wave) * kUGroup + k0 % kUGroup;
    if (c0 >= nchunks) break;
    // the lane's chunk; chunks past the end re-read the last one and are not accumulated
    const int64_t col = min(c0 + lp / 4, nchunks - 1) * 32;
    u32x4 xv[16 / RI], av[NT][16 / RI];
#pragma unroll
    for (int i = 0; i < 16 / RI; ++i) xv[i] = *reinterpret_cast<const u32x4*>(xsrc[i] + col);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16 / RI; ++i)
        av[t][i] = *reinterpret_cast<const u32x4*>(ut.A[t] + (int64_t)RI * i * K + aoff + col);
    __builtin_amdgcn_wave_barrier();   // the previous batch's slice reads come first
#pragma unroll
    for (int i = 0; i < 16 / RI; ++i) {
      slice[slot(0, RI * i + lane / P, lp)] = xv[i];
#pragma unroll
      for (int t = 0; t < NT; ++t) slice[slot(1 + t, RI * i + lane / P, lp)] = av[t][i];
    }
    __builtin_amdgcn_wave_barrier();   // the slice is written before it is read
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int m = lane & 15, p = 4 * b + (lane >> 4);
      const u32x4 xo = slice[slot(0, m, p)];
      u32x4 ao[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) ao[t] = slice[slot(1 + t, m, p)];
      if (c0 + b < nchunks) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xo), __builtin_bit_cast(bf16x8, ao[t]),
                                                           acc[t], 0, 0, 0);
      }
    }
  }
  __syncthreads();   // every wave is done with its slice; the space now holds the waves' sums
  f32x4* red = reinterpret_cast<f32x4*>(lds);   // [wave][t][lane]
#pragma unroll
  for (int t = 0; t < NT; ++t) red[(wave * NT + t) * 64 + lane] = acc[t];
  __syncthreads();
  // output o = (row, j): acc[t][i] of lane (row / 4) * 16 + j % 16 holds row 4 (lane / 16) + i
  for (int o = tid; o < 16 * r; o += kUWaves * 64) {
    const int row = o / r, j = o % r;
    const int t = j >> 4, ln = (row >> 2) * 16 + (j & 15), i = row & 3;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kUWaves; ++w) v += red[(w * NT + t) * 64 + ln][i];
    if (m0 + row < M) {
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
        if (tt == t) ut.u[tt][(m0 + row) * ut.ustride + (j & 15)] = v;
    }
  }
}

bool lora_u_uses_pass(int r) { return r > 16; }

static void launch_u_tiles(const uint16_t* X, int64_t M, int64_t K, int nt, const UTiles& ut, hipStream_t stream) {
  const dim3 grid((unsigned)((M + 15) / 16)), block(kUWaves * 64);
  switch (nt) {
    case 1: hipLaunchKernelGGL(lora_u_kernel<1>, grid, block, 0, stream, X, M, K, ut); break;
    case 2: hipLaunchKernelGGL(lora_u_kernel<2>, grid, block, 0, stream, X, M, K, ut); break;
    case 3: hipLaunchKernelGGL(lora_u_kernel<3>, grid, block, 0, stream, X, M, K, ut); break;
    case 4: hipLaunchKernelGGL(lora_u_kernel<4>, grid, block, 0, stream, X, M, K, ut); break;
    case 5: hipLaunchKernelGGL(lora_u_kernel<5>, grid, block, 0, stream, X, M, K, ut); break;
    case 6: hipLaunchKernelGGL(lora_u_kernel<6>, grid, block, 0, stream, X, M, K, ut); break;
    case 7: hipLaunchKernelGGL(lora_u_kernel<7>, grid, block, 0, stream, X, M, K, ut); break;
    default: hipLaunchKernelGGL(lora_u_kernel<8>, grid, block, 0, stream, X, M, K, ut); break;
  }
}

hipError_t launch_lora_u_group(const uint16_t* X, int64_t M, int64_t K, int count, const uint16_t* const* A,
                               float* const* u, hipStream_t stream) {
  if (count < 1 || count > 8) return hipErrorInvalidValue;
  UTiles ut{};
  for (int i = 0; i < count; ++i) {
    ut.A[i] = A[i];
    ut.u[i] = u[i];
  }
  ut.ustride = 16;
  launch_u_tiles(X, M, K, count, ut, stream);
  return hipGetLastError();
}

hipError_t launch_lora_u(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A, int r,
                         float* ws, float* u, hipStream_t stream) {
  if (lora_u_uses_pass(r)) {
    // above rank 16 a workgroup of lora_u_kernel would read r x K of A for its 16 rows: the pass
    // reads A once per row block of 256 and leaves partial sums over column ranges in ws
    const LoraPassPlan p = lora_pass_plan(M, K, r);
    const LoraPassArgs a{X, M, K, A, {}, r, r, p.crange, ws, nullptr, 0};
    launch_pass<true, false, false>(p, a, stream);
    const ReduceJob j = reduce_job(ws, p.cranges, M * r, 0, r, false, 1.f, 0, u);
    launch_reduce(&j, 1, stream);
    return hipGetLastError();
  }
  UTiles ut{};
  for (int t = 0; t < r / 16; ++t) {
    ut.A[t] = A + (int64_t)t * 16 * K;
    ut.u[t] = u + 16 * t;
  }
  ut.ustride = r;
  launch_u_tiles(X, M, K, r / 16, ut, stream);
  return hipGetLastError();
}

size_t lora_dy_group_ws_floats(int count, const int64_t* N, int64_t M, int r) {
  size_t f = 0;
  for (int i = 0; i < count; ++i) f += lora_pass_ws_floats(M, N[i], r, true, true);
  return f;
}

hipError_t launch_lora_dy_group(int count, const LoraDyItem* it, int64_t M, int r, float scale, int accumulate,
                                float* ws, hipStream_t stream) {
  if (count < 1 || count > kMaxPassGroup || 2 * count > kMaxReduceJobs) return hipErrorInvalidValue;
  ReduceJob jobs[kMaxReduceJobs];
  LoraPassPlan p[kMaxPassGroup];
  LoraPassArgs a[kMaxPassGroup];
  for (int i = 0; i < count; ++i) {
    p[i] = lora_pass_plan(M, it[i].N, r);
    float* part_down = ws;
    float* part_grad = ws + (size_t)p[i].cranges * M * r;
    ws = part_grad + (size_t)p[i].mblocks * it[i].N * r;
    a[i] = LoraPassArgs{it[i].dY, M, it[i].N, it[i].B, {it[i].u}, r, r, p[i].crange, part_down, part_grad, 0};
    jobs[2 * i] = reduce_job(part_down, p[i].cranges, M * r, 0, r, false, 1.f, 0, it[i].v);
    jobs[2 * i + 1] = reduce_job(part_grad, p[i].mblocks, it[i].N * r, 0, r, false, scale, accumulate, it[i].dB);
  }
  launch_passes<true, true, true>(count, p, a, stream);
  launch_reduce(jobs, 2 * count, stream);
  return hipGetLastError();
}

hipError_t launch_lora_dy(const uint16_t* dY, int64_t M, int64_t N, const uint16_t* B, const float* u,
                          int r, float scale, int accumulate, float* ws, float* v, float* dB,
                          hipStream_t stream) {
  const LoraDyItem it{dY, N, B, u, v, dB};
  return launch_lora_dy_group(1, &it, M, r, scale, accumulate, ws, stream);
}

// The passes over X of linears that share it take one launch while their ranks add up to 64 or less:
// the grad operands then sit side by side in the pass's tiles and the row blocks stay 256 rows, so
// each dA comes out as its own pass would give it, bit for bit.
static bool dx_pass_grouped(int count, int r) { return count > 1 && count * r <= 64; }

size_t lora_dx_group_ws_floats(int count, int64_t M, int64_t K, int r) {
  return dx_pass_grouped(count, r) ? lora_pass_ws_floats(M, K, count * r, false, true)
                                   : (size_t)count * lora_pass_ws_floats(M, K, r, false, true);
}

hipError_t launch_lora_dx_group(int count, const uint16_t* X, int64_t M, int64_t K, const float* const* v, int r,
                                float scale, int accumulate, float* ws, float* const* dA, hipStream_t stream) {
  if (count < 1 || count > 4) return hipErrorInvalidValue;
  ReduceJob jobs[4];
  if (dx_pass_grouped(count, r)) {
    const LoraPassPlan p = lora_pass_plan(M, K, count * r);
    LoraPassArgs a{X, M, K, nullptr, {}, r, count * r, p.crange, nullptr, ws, 0};
    for (int i = 0; i < count; ++i) a.P[i] = v[i];
    launch_pass<false, true, false>(p, a, stream);
    for (int i = 0; i < count; ++i)
      jobs[i] = reduce_job(ws + (size_t)i * p.mblocks * K * r, p.mblocks, K * r, K, r, true, scale, accumulate, dA[i]);
  } else {
    // one pass per linear, all in one launch
    LoraPassPlan p[kMaxPassGroup];
    LoraPassArgs a[kMaxPassGroup];
    for (int i = 0; i < count; ++i) {
      p[i] = lora_pass_plan(M, K, r);
      a[i] = LoraPassArgs{X, M, K, nullptr, {v[i]}, r, r, p[i].crange, nullptr, ws, 0};
      jobs[i] = reduce_job(ws, p[i].mblocks, K * r, K, r, true, scale, accumulate, dA[i]);
      ws += (size_t)p[i].mblocks * K * r;
    }
    launch_passes<false, true, false>(count, p, a, stream);
  }
  launch_reduce(jobs, count, stream);
  return hipGetLastError();
}

hipError_t launch_lora_dx(const uint16_t* X, int64_t M, int64_t K, const float* v, int r, float scale,
                          int accumulate, float* ws, float* dA, hipStream_t stream) {
  return launch_lora_dx_group(1, X, M, K, &v, r, scale, accumulate, ws, &dA, stream);
}

}  // namespace nf4
