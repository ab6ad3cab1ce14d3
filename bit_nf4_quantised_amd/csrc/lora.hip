// Adapter (LoRA) kernels of the adapted linear (gfx950).
//
// "QLoRA, explained", The forward pass and gradients: the adapter gradients are LoRA's with the
// dequantised weight in place of the original, dB = s G A^T and dA = s B^T G with G = dY^T X.
// Computed here without forming G (N x K):
//   u  = X A^T   [M x r]   (forward; saved for the backward)
//   v  = dY B    [M x r]   (backward)
//   dA = s v^T X [r x K]   and   dB = s dY^T u [N x r]     (fp32, optionally accumulated)
// All reductions run in a fixed order (no atomics), so results are bitwise reproducible.
#include "common.h"
#include "launch.h"

namespace nf4 {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

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

// ------------------------------------------------------------------------------------------
// Partial down-projection: part[c][m][j] = sum over l in chunk c of P[m][l] * Q(j, l), where
// Q(j, l) = A[j][l] (A is r x L, QT = false) or B[l][j] (B is L x r, QT = true).
// Workgroup: 64 activation rows (16 per wave) x one contraction chunk.
template <bool QT>
__global__ __launch_bounds__(256) void lora_down_kernel(const uint16_t* __restrict__ P, int64_t M,
                                                        int64_t L, const uint16_t* __restrict__ Q,
                                                        int r, int64_t chunk_len,
                                                        float* __restrict__ part) {
  constexpr int QP = 128 + 8;  // staged Q rows hold up to 128 rank columns
  __shared__ __attribute__((aligned(16))) uint16_t Qs[4][32][QP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m = (int64_t)blockIdx.x * 64 + wave * 16 + (lane & 15);
  const int chunk = blockIdx.y;
  const int64_t l_begin = (int64_t)chunk * chunk_len;
  const int64_t l_end = min(L, l_begin + chunk_len);
  const int RT = r / 16;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t l0 = l_begin; l0 < l_end; l0 += 32) {
    const int64_t l = l0 + 8 * (lane >> 4);
    bf16x8 b = {};
    if (m < M && l < l_end) b = *reinterpret_cast<const bf16x8*>(P + m * L + l);
    if (QT) {
      // stage B rows l0 .. l0+31 (r columns each) for this wave
      const int cols8 = r / 8;
      for (int q = lane; q < 32 * cols8; q += 64) {
        const int row = q / cols8, c8 = (q % cols8) * 8;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (l0 + row < l_end) v = *reinterpret_cast<const u32x4*>(Q + (l0 + row) * r + c8);
        *reinterpret_cast<u32x4*>(&Qs[wave][row][c8]) = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      if (jt < RT) {
        bf16x8 a;
        if (QT) {
          a = tr_frag(&Qs[wave][0][0], QP, jt * 16, lane);
        } else {
          a = bf16x8{};
          if (l < l_end) a = *reinterpret_cast<const bf16x8*>(Q + (int64_t)(jt * 16 + (lane & 15)) * L + l);
        }
        acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[jt], 0, 0, 0);
      }
    }
    if (QT) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  if (m < M) {
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      if (jt < RT) {
        const int j = jt * 16 + 4 * (lane >> 4);
        *reinterpret_cast<f32x4*>(part + ((int64_t)chunk * M + m) * r + j) = acc[jt];
      }
    }
  }
}

// out[m][j] = sum over chunks, in chunk order.
__global__ __launch_bounds__(256) void lora_down_reduce_kernel(const float* __restrict__ part,
                                                               int nchunks, int64_t count,
                                                               float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float s = 0.f;
  for (int c = 0; c < nchunks; ++c) s += part[(int64_t)c * count + i];
  out[i] = s;
}

// ------------------------------------------------------------------------------------------
// Adapter gradients: D[c][j] = sum_m Q[m][c] * P[m][j] with P fp32 [M x r] split into bf16
// hi + lo parts (P - hi rounded again), Q bf16 [M x C].
//   OUT_CR = false: out is [r x C] (dA = s v^T X: P = v, Q = X)
//   OUT_CR = true:  out is [C x r] (dB = s dY^T u: P = u, Q = dY)
// Workgroup (blockIdx.x, blockIdx.y) = (64 columns c, one slice of M). Its four waves take
// interleaved 32-row slices of that range, prefetching the next slice into registers while the
// current one is multiplied; the waves are summed in wave order into part[slice][c][j], and
// lora_grad_reduce_kernel sums the slices in order, scales and writes (or accumulates) the output.
template <bool OUT_CR>
__global__ __launch_bounds__(256) void lora_grad_kernel(const float* __restrict__ P,
                                                        const uint16_t* __restrict__ Q, int64_t M,
                                                        int64_t C, int r, int64_t m_per_slice,
                                                        float* __restrict__ part) {
  constexpr int QP = 64 + 8, PP = 128 + 8, RP = 128 + 1;
  constexpr int kStage = 4 * 32 * QP * 2 + 2 * 4 * 32 * PP * 2;
  constexpr int kRed = 4 * 64 * RP * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStage > kRed ? kStage : kRed];
  auto Qs = reinterpret_cast<uint16_t(*)[32][QP]>(smem);
  auto Ph = reinterpret_cast<uint16_t(*)[32][PP]>(smem + 4 * 32 * QP * 2);
  auto Pl = reinterpret_cast<uint16_t(*)[32][PP]>(smem + 4 * 32 * QP * 2 + 4 * 32 * PP * 2);
  auto Red = reinterpret_cast<float(*)[64][RP]>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  const int64_t m_begin = (int64_t)blockIdx.y * m_per_slice;
  const int64_t m_end = min(M, m_begin + m_per_slice);
  const int RT = r / 16;
  const int cols4 = r / 4;             // float4 chunks per P row
  const int pchunks = 32 * cols4 / 64; // float4 chunks of a 32-row P slice per lane (2 .. 16)
  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 qreg[4];
  f32x4 preg[16];
  auto load = [&](int64_t mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = lane + 64 * i;
      const int row = q >> 3, c8 = (q & 7) * 8;
      qreg[i] = (mb + row < m_end && c0 + c8 < C)
                    ? *reinterpret_cast<const u32x4*>(Q + (mb + row) * C + c0 + c8)
                    : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < pchunks) {
        const int q = lane + 64 * i;
        const int row = q / cols4, c4 = (q % cols4) * 4;
        preg[i] = (mb + row < m_end) ? *reinterpret_cast<const f32x4*>(P + (mb + row) * r + c4)
                                     : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = lane + 64 * i;
      *reinterpret_cast<u32x4*>(&Qs[wave][q >> 3][(q & 7) * 8]) = qreg[i];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < pchunks) {
        const int q = lane + 64 * i;
        const int row = q / cols4, c4 = (q % cols4) * 4;
        const f32x4 v = preg[i];
        const uint32_t h01 = pack_bf16x2(v[0], v[1]), h23 = pack_bf16x2(v[2], v[3]);
        const uint32_t l01 = pack_bf16x2(v[0] - __uint_as_float(h01 << 16),
                                         v[1] - __uint_as_float(h01 & 0xFFFF0000u));
        const uint32_t l23 = pack_bf16x2(v[2] - __uint_as_float(h23 << 16),
                                         v[3] - __uint_as_float(h23 & 0xFFFF0000u));
        *reinterpret_cast<u32x2*>(&Ph[wave][row][c4]) = u32x2{h01, h23};
        *reinterpret_cast<u32x2*>(&Pl[wave][row][c4]) = u32x2{l01, l23};
      }
    }
  };

  // uniform trip count across waves: every wave runs `rounds` rounds (empty slices are zeros)
  const int64_t rows = m_end > m_begin ? m_end - m_begin : 0;
  const int64_t rounds = (rows + 127) / 128;
  if (rounds > 0) load(m_begin + wave * 32);
  for (int64_t rd = 0; rd < rounds; ++rd) {
    stage();
    if (rd + 1 < rounds) load(m_begin + ((rd + 1) * 4 + wave) * 32);
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const bf16x8 qf = tr_frag(&Qs[wave][0][0], QP, ct * 16, lane);
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) {
        if (rt < RT) {
          const bf16x8 ph = tr_frag(&Ph[wave][0][0], PP, rt * 16, lane);
          const bf16x8 pl = tr_frag(&Pl[wave][0][0], PP, rt * 16, lane);
          if (OUT_CR) {
            acc[ct][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, qf, acc[ct][rt], 0, 0, 0);
            acc[ct][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, qf, acc[ct][rt], 0, 0, 0);
          } else {
            acc[ct][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf, ph, acc[ct][rt], 0, 0, 0);
            acc[ct][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf, pl, acc[ct][rt], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
  }
  // acc[ct][rt][i]: OUT_CR = false: c = ct*16 + 4*(lane/16) + i, j = rt*16 + lane%16
  //                 OUT_CR = true:  j = rt*16 + 4*(lane/16) + i, c = ct*16 + lane%16
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
      if (rt < RT)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int c, j;
          if (OUT_CR) { j = rt * 16 + 4 * (lane >> 4) + i; c = ct * 16 + (lane & 15); }
          else        { c = ct * 16 + 4 * (lane >> 4) + i; j = rt * 16 + (lane & 15); }
          Red[wave][c][j] = acc[ct][rt][i];
        }
  __syncthreads();
  // part[slice][c][j] for the 64 columns of this workgroup
  float* dst = part + (int64_t)blockIdx.y * C * r;
  for (int idx = tid; idx < 64 * r; idx += 256) {
    const int c = idx / r, j = idx % r;
    const int64_t cc = c0 + c;
    if (cc < C) dst[cc * r + j] = ((Red[0][c][j] + Red[1][c][j]) + Red[2][c][j]) + Red[3][c][j];
  }
}

// out = scale * sum over slices (in slice order) [+ out]; out is [C x r] (OUT_CR) or [r x C].
__global__ __launch_bounds__(256) void lora_grad_reduce_kernel(const float* __restrict__ part,
                                                               int slices, int64_t C, int r,
                                                               float scale, int out_cr,
                                                               float* __restrict__ out,
                                                               int accumulate) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = C * r;
  if (idx >= total) return;
  // idx walks the output in memory order
  int64_t c, j;
  if (out_cr) { c = idx / r; j = idx % r; }
  else        { j = idx / C; c = idx % C; }
  float v = 0.f;
  for (int sl = 0; sl < slices; ++sl) v += part[(int64_t)sl * total + c * r + j];
  v *= scale;
  out[idx] = accumulate ? out[idx] + v : v;
}

// ------------------------------------------------------------------------------------------
// Contraction chunking of the down-projection: about 512 workgroups, chunks of whole 32-column
// steps, at least 256 columns each. Returns the chunk count and sets the chunk length.
static int lora_down_plan(int64_t M, int64_t L, int64_t* chunk_len) {
  const int64_t mtiles = (M + 63) / 64;
  int64_t want = (512 + mtiles - 1) / mtiles;
  const int64_t maxc = (L + 255) / 256;
  if (want > maxc) want = maxc;
  if (want < 1) want = 1;
  *chunk_len = ((L + want - 1) / want + 31) / 32 * 32;
  return (int)((L + *chunk_len - 1) / *chunk_len);
}

int lora_down_chunks(int64_t M, int64_t L) {
  int64_t len;
  return lora_down_plan(M, L, &len);
}

hipError_t launch_lora_down(const uint16_t* P, int64_t M, int64_t L, const uint16_t* Q, bool q_is_lr,
                            int r, float* part, float* out, hipStream_t stream) {
  int64_t chunk_len;
  const int nchunks = lora_down_plan(M, L, &chunk_len);
  dim3 grid((unsigned)((M + 63) / 64), (unsigned)nchunks);
  if (q_is_lr)
    hipLaunchKernelGGL((lora_down_kernel<true>), grid, dim3(256), 0, stream, P, M, L, Q, r, chunk_len, part);
  else
    hipLaunchKernelGGL((lora_down_kernel<false>), grid, dim3(256), 0, stream, P, M, L, Q, r, chunk_len, part);
  const int64_t count = M * r;
  hipLaunchKernelGGL(lora_down_reduce_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                     stream, part, nchunks, count, out);
  return hipGetLastError();
}

// Token slices of the gradient kernels: about 512 workgroups, slices of whole 128-row rounds.
static int lora_grad_plan(int64_t M, int64_t C, int64_t* m_per_slice) {
  const int64_t ctiles = (C + 63) / 64;
  int64_t want = (512 + ctiles - 1) / ctiles;
  const int64_t maxs = (M + 127) / 128;
  if (want > maxs) want = maxs;
  if (want < 1) want = 1;
  *m_per_slice = ((M + want - 1) / want + 127) / 128 * 128;
  return (int)((M + *m_per_slice - 1) / *m_per_slice);
}

size_t lora_grad_workspace_floats(int64_t M, int64_t C, int r) {
  int64_t mps;
  return (size_t)lora_grad_plan(M, C, &mps) * (size_t)C * (size_t)r;
}

hipError_t launch_lora_grad(const float* P, const uint16_t* Q, int64_t M, int64_t C, int r,
                            float scale, float* out, bool out_cr, int accumulate, float* part,
                            hipStream_t stream) {
  int64_t mps;
  const int slices = lora_grad_plan(M, C, &mps);
  dim3 grid((unsigned)((C + 63) / 64), (unsigned)slices);
  if (out_cr)
    hipLaunchKernelGGL((lora_grad_kernel<true>), grid, dim3(256), 0, stream, P, Q, M, C, r, mps, part);
  else
    hipLaunchKernelGGL((lora_grad_kernel<false>), grid, dim3(256), 0, stream, P, Q, M, C, r, mps, part);
  const int64_t total = C * r;
  hipLaunchKernelGGL(lora_grad_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     stream, part, slices, C, r, scale, out_cr ? 1 : 0, out, accumulate);
  return hipGetLastError();
}

}  // namespace nf4
