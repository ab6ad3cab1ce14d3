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
// A workgroup takes 256 (or, above rank 32, 128) rows and a range of columns, streaming 64-column
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
  const float* P;           // grad operand [M x r] fp32
  int r;
  int64_t crange;           // columns per workgroup column range (a multiple of kStepC)
  float* part_down;         // [column ranges][M][r]
  float* part_grad;         // [row blocks][C][r]
};

// R16: the rank is exactly 16 (the common case): the grad operand fragments stay in registers.
template <int MB, bool DOWN, bool GRAD, bool RT, bool R16>
__global__ __launch_bounds__(256) void lora_pass_kernel(const LoraPassArgs a) {
  constexpr int QS = MB == 256 ? 3 : 2;                 // Q stages in LDS
  constexpr int NQ = MB / 32;                           // Q DMA loads per wave per step
  constexpr int RMAX = MB == 256 ? 32 : 128;            // largest rank handled
  constexpr int RTILE = DOWN ? kStepC * RMAX : 8;       // R tile elements per stage
  constexpr int PP = (GRAD ? RMAX : 0) + 8;             // pitch of the P tiles
  __shared__ __attribute__((aligned(16))) uint16_t Qs[QS][MB * kStepC];
  __shared__ __attribute__((aligned(16))) uint16_t Rs[QS][RTILE];
  __shared__ __attribute__((aligned(16))) uint16_t Ph[GRAD ? MB : 1][PP];
  __shared__ __attribute__((aligned(16))) uint16_t Pl[GRAD ? MB : 1][PP];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = R16 ? 16 : a.r, RT16 = r / 16;
  const int64_t m0 = (int64_t)blockIdx.x * MB;
  const int64_t rows_valid = min(a.M - m0, (int64_t)MB);
  const int64_t c_begin = (int64_t)blockIdx.y * a.crange;
  const int64_t c_end = min(a.C, c_begin + a.crange);
  const int nsteps = (int)((c_end - c_begin + kStepC - 1) / kStepC);

  // ---- DMA of one step: Q rows m0.., columns c0 .. c0+63 (swizzled), then the R tile
  const int rdma = (r + 31) / 32;   // R loads per wave per step (waves past the tile repeat one)
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
      f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
      if (row < rows_valid) v = *reinterpret_cast<const f32x4*>(a.P + (m0 + row) * r + c4);
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
        float* dst = a.part_grad + ((int64_t)blockIdx.x * a.C + c) * r + 4 * (lane >> 4);
#pragma unroll
        for (int jt = 0; jt < RMAX / 16; ++jt)
          if (jt < RT16) *reinterpret_cast<f32x4*>(dst + jt * 16) = gacc[jt];
      }
    }
  };

  // ---- pipeline: QS-1 steps in flight. Step t: start the DMA of step t+QS-1, wait until step
  // t's loads have landed (later steps' loads may stay in flight: vector-memory loads complete in
  // issue order), barrier, compute, barrier (the stage is refilled next).
  const int per_step = NQ + (DOWN ? rdma : 0);
  for (int t = 0; t < QS - 1 && t < nsteps; ++t) issue(t);
  for (int t = 0; t < nsteps; ++t) {
    if (t + QS - 1 < nsteps) {
      issue(t + QS - 1);
      // allowance: the loads of steps t+1 .. t+QS-1
      if (QS == 3) {
        if (per_step == NQ) wait_vmcnt<2 * NQ>();
        else if (per_step == NQ + 1) wait_vmcnt<2 * (NQ + 1)>();
        else if (per_step == NQ + 2) wait_vmcnt<2 * (NQ + 2)>();
        else wait_vmcnt<0>();
      } else {
        if (per_step == NQ) wait_vmcnt<NQ>();
        else if (per_step == NQ + 1) wait_vmcnt<NQ + 1>();
        else if (per_step == NQ + 2) wait_vmcnt<NQ + 2>();
        else if (per_step == NQ + 3) wait_vmcnt<NQ + 3>();
        else if (per_step == NQ + 4) wait_vmcnt<NQ + 4>();
        else wait_vmcnt<0>();
      }
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    compute(t);
    lds_barrier();
  }

  if (DOWN) {
    float* dst = a.part_down + (int64_t)blockIdx.y * a.M * r;
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
// serves two jobs (blocks [0, blocks0) take job 0). A thread takes one output and issues the loads
// of 8 partials at a time before adding them in order; the sums are latency-bound chains, so
// one output per thread gives the most chains in flight.
struct ReduceJob {
  const float* part;
  int nparts;
  int64_t count, C;
  int r, transpose, accumulate;
  float scale;
  float* out;
};

__global__ __launch_bounds__(256) void lora_reduce_kernel(const ReduceJob j0, const ReduceJob j1, int blocks0) {
  const bool second = (int)blockIdx.x >= blocks0;
  const ReduceJob& jb = second ? j1 : j0;
  const int64_t i = (int64_t)(second ? blockIdx.x - blocks0 : blockIdx.x) * 256 + threadIdx.x;
  if (i >= jb.count) return;
  const int64_t src = jb.transpose ? (i % jb.C) * jb.r + i / jb.C : i;
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
// Work split of a pass: row blocks of 256 (128 above rank 32) and column ranges of whole steps,
// about 256 workgroups in all with at least 4 steps per workgroup where the matrix allows it.
LoraPassPlan lora_pass_plan(int64_t M, int64_t C, int r) {
  LoraPassPlan p;
  p.mb = r > 32 ? 128 : 256;
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

template <bool DOWN, bool GRAD, bool RT>
static void launch_pass(const LoraPassPlan& p, const LoraPassArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)p.mblocks, (unsigned)p.cranges);
  if (p.mb == 256 && a.r == 16)
    hipLaunchKernelGGL((lora_pass_kernel<256, DOWN, GRAD, RT, true>), grid, dim3(256), 0, stream, a);
  else if (p.mb == 256)
    hipLaunchKernelGGL((lora_pass_kernel<256, DOWN, GRAD, RT, false>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((lora_pass_kernel<128, DOWN, GRAD, RT, false>), grid, dim3(256), 0, stream, a);
}

static ReduceJob reduce_job(const float* part, int nparts, int64_t count, int64_t C, int r, bool transpose,
                            float scale, int accumulate, float* out) {
  return ReduceJob{part, nparts, count, C, r, transpose ? 1 : 0, accumulate, scale, out};
}

static void launch_reduce(const ReduceJob& j0, const ReduceJob* j1, hipStream_t stream) {
  const int b0 = (int)((j0.count + 255) / 256);
  const int b1 = j1 ? (int)((j1->count + 255) / 256) : 0;
  hipLaunchKernelGGL(lora_reduce_kernel, dim3((unsigned)(b0 + b1)), dim3(256), 0, stream, j0, j1 ? *j1 : j0, b0);
}

// ------------------------------------------------------------------------------------------
// u = X A^T in one launch, without partial sums in memory (its contraction runs over K only, so
// a workgroup can own whole rows): a workgroup owns 16 rows of X and all of K. Its 8 waves take
// interleaved 32-column chunks (wave w: chunks w, w + 8, ...), NB chunks at a time with every
// load of a batch issued before its MFMAs; lane (row = lane % 16, g = lane / 16) holds columns
// 8 g .. 8 g + 7 of the chunk of its row of X and of row 16 t + lane % 16 of A for each 16-row
// tile t of A, and v_mfma_f32_16x16x32_bf16 accumulates u[row][16 t + j]. The workgroup then sums
// the 8 waves in LDS in wave order.
constexpr int kUWaves = 8;

template <int NT>   // r / 16
__global__ __launch_bounds__(kUWaves * 64) void lora_u_kernel(const uint16_t* __restrict__ X, int64_t M,
                                                            int64_t K, const uint16_t* __restrict__ A,
                                                            float* __restrict__ u) {
  constexpr int NB = NT >= 8 ? 1 : 8 / NT;   // chunks per batch
  constexpr int r = 16 * NT;
  __shared__ f32x4 red[kUWaves][NT][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  const uint16_t* xrow = X + min(m0 + (lane & 15), M - 1) * K + 8 * g;
  const uint16_t* arow = A + (int64_t)(lane & 15) * K + 8 * g;
  const int64_t nchunks = K / 32;

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t c0 = wave; c0 < nchunks; c0 += (int64_t)kUWaves * NB) {
    bf16x8 xv[NB], av[NB][NT];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      // chunks past the end re-read the last one and are not accumulated
      const int64_t col = min(c0 + (int64_t)kUWaves * b, nchunks - 1) * 32;
      xv[b] = *reinterpret_cast<const bf16x8*>(xrow + col);
#pragma unroll
      for (int t = 0; t < NT; ++t) av[b][t] = *reinterpret_cast<const bf16x8*>(arow + (int64_t)t * 16 * K + col);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (c0 + (int64_t)kUWaves * b < nchunks) {
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv[b], av[b][t], acc[t], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  // output o = (row, j): acc[t][i] of lane (row / 4) * 16 + j % 16 holds row 4 (lane / 16) + i
  for (int o = tid; o < 16 * r; o += kUWaves * 64) {
    const int row = o / r, j = o % r;
    const int t = j >> 4, ln = (row >> 2) * 16 + (j & 15), i = row & 3;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kUWaves; ++w) v += red[w][t][ln][i];
    if (m0 + row < M) u[(m0 + row) * r + j] = v;
  }
}

hipError_t launch_lora_u(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A, int r,
                         float* ws, float* u, hipStream_t stream) {
  (void)ws;
  const dim3 grid((unsigned)((M + 15) / 16)), block(kUWaves * 64);
  switch (r / 16) {
    case 1: hipLaunchKernelGGL(lora_u_kernel<1>, grid, block, 0, stream, X, M, K, A, u); break;
    case 2: hipLaunchKernelGGL(lora_u_kernel<2>, grid, block, 0, stream, X, M, K, A, u); break;
    case 3: hipLaunchKernelGGL(lora_u_kernel<3>, grid, block, 0, stream, X, M, K, A, u); break;
    case 4: hipLaunchKernelGGL(lora_u_kernel<4>, grid, block, 0, stream, X, M, K, A, u); break;
    case 5: hipLaunchKernelGGL(lora_u_kernel<5>, grid, block, 0, stream, X, M, K, A, u); break;
    case 6: hipLaunchKernelGGL(lora_u_kernel<6>, grid, block, 0, stream, X, M, K, A, u); break;
    case 7: hipLaunchKernelGGL(lora_u_kernel<7>, grid, block, 0, stream, X, M, K, A, u); break;
    default: hipLaunchKernelGGL(lora_u_kernel<8>, grid, block, 0, stream, X, M, K, A, u); break;
  }
  return hipGetLastError();
}

hipError_t launch_lora_dy(const uint16_t* dY, int64_t M, int64_t N, const uint16_t* B, const float* u,
                          int r, float scale, int accumulate, float* ws, float* v, float* dB,
                          hipStream_t stream) {
  const LoraPassPlan p = lora_pass_plan(M, N, r);
  float* part_down = ws;
  float* part_grad = ws + (size_t)p.cranges * M * r;
  LoraPassArgs a{dY, M, N, B, u, r, p.crange, part_down, part_grad};
  launch_pass<true, true, true>(p, a, stream);
  const ReduceJob jv = reduce_job(part_down, p.cranges, M * r, 0, r, false, 1.f, 0, v);
  const ReduceJob jb = reduce_job(part_grad, p.mblocks, N * r, 0, r, false, scale, accumulate, dB);
  launch_reduce(jv, &jb, stream);
  return hipGetLastError();
}

hipError_t launch_lora_dx(const uint16_t* X, int64_t M, int64_t K, const float* v, int r, float scale,
                          int accumulate, float* ws, float* dA, hipStream_t stream) {
  const LoraPassPlan p = lora_pass_plan(M, K, r);
  LoraPassArgs a{X, M, K, nullptr, v, r, p.crange, nullptr, ws};
  launch_pass<false, true, false>(p, a, stream);
  launch_reduce(reduce_job(ws, p.mblocks, K * r, K, r, true, scale, accumulate, dA), nullptr, stream);
  return hipGetLastError();
}

}  // namespace nf4
