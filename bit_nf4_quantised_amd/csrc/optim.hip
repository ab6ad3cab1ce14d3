// The adapter update of a training step (gfx950): global gradient-norm clipping, then AdamW.
//
// "QLoRA, explained", The algorithm, step by step / Minimal implementation: after the backward the
// adapter gradients are clipped by their global norm (0.3 in the original runs) and AdamW (32-bit state)
// updates A and B only. AdamW with decoupled weight decay, for clipped gradient g at step t:
//   p <- p (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;
//   p <- p - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps)
// with master weights and moments in fp32, and an optional bf16 copy of the new weights for the
// next forward (round to nearest even).
//
// A plan holds, in device memory, one 48-byte descriptor per 4096-value chunk of every tensor
// (the five pointers already offset to the chunk, and its length), built once on the host, so a
// step over any number of tensors is three launches whatever their count:
//   1. squared-norm partial sums in double, a fixed grid of at most 1024 workgroups striding over
//      the chunks;
//   2. one workgroup adds the partial sums (every sum in a fixed order: bitwise reproducible);
//   3. the elementwise update, one workgroup per chunk, reading the norm from step 2.
// The norm must be complete before any element changes, hence the separate passes. Bound by
// HBM: per value the norm reads 4 bytes, the update reads 16 (p, g, m, v) and writes 12 (p, m, v)
// plus 2 for the bf16 copy.
#include <stdlib.h>

#include "common.h"
#include "launch.h"

namespace nf4 {

constexpr int kOptChunk = 4096;      // values per update workgroup: 256 threads x 4 float4
constexpr int kOptNormGrid = 1024;   // workgroups of the norm's partial sums (fewer if fewer chunks)

struct OptChunk {                    // one chunk of one tensor; pointers already offset
  float* p;
  const float* g;
  float* m;
  float* v;
  uint16_t* pb;                      // may be null
  int64_t len;                       // values in the chunk: a multiple of 4 in 4..4096
};
static_assert(sizeof(OptChunk) == 48, "descriptor layout");

struct OptScalars {
  float beta1, beta2, eps, decay;    // decay = 1 - lr * weight_decay
  float step_size, inv_sqrt_bc2;     // lr / (1 - b1^t), 1 / sqrt(1 - b2^t)
  float max_norm;                    // <= 0: no clipping
};

// The table's pointers arrive as generic pointers; naming them global lets the loads and stores
// use the global (not flat) instructions, which do not tie up the scalar/LDS wait counter.
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* as_global(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

// Sum over the 256 threads of a workgroup in a fixed order (butterfly within each wave, then the
// four wave sums pairwise); every thread receives the total.
__device__ __forceinline__ double block_sum(double x, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Loads of one chunk for the norm: four 16-byte loads per thread. A chunk index past the end of
// the table reads the table's last chunk with length 0 (its values are then ignored).
__device__ __forceinline__ void norm_load(const OptChunk* __restrict__ table, int c, int chunks,
                                          f32x4 (&x)[kOptChunk / 1024], int64_t& len) {
  const int cc = c < chunks ? c : chunks - 1;
  const float* g = table[cc].g;
  len = c < chunks ? table[cc].len : 0;
  const int64_t last = len > 0 ? len - 4 : 0;
#pragma unroll
  for (int i = 0; i < kOptChunk / 1024; ++i) {
    const int64_t e = 4 * ((int64_t)threadIdx.x + 256 * i);
    x[i] = *as_global(reinterpret_cast<const f32x4*>(g + (e < len ? e : last)));
  }
}

__device__ __forceinline__ double norm_sum(const f32x4 (&x)[kOptChunk / 1024], int64_t len) {
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kOptChunk / 1024; ++i) {
    const int64_t e = 4 * ((int64_t)threadIdx.x + 256 * i);
    double q = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k) q += (double)x[i][k] * (double)x[i][k];
    s += e < len ? q : 0.0;
  }
  return s;
}

// Partial sums of squares over a fixed grid of G workgroups: workgroup w takes chunks w, w + G,
// w + 2G, ... in that order, with the next chunk's loads in flight while the current one is
// summed (two fixed register slots). Every sum's order depends only on G and the table.
__global__ __launch_bounds__(256) void grad_sqnorm_partial_kernel(const OptChunk* __restrict__ table,
                                                                  int chunks, double* partial) {
  __shared__ double red[4];
  const int G = gridDim.x;
  const int trips = (chunks - (int)blockIdx.x + G - 1) / G;   // >= 1: the grid is at most chunks
  f32x4 a[kOptChunk / 1024], b[kOptChunk / 1024];
  int64_t la, lb;
  int c = blockIdx.x;
  norm_load(table, c, chunks, a, la);
  double s = 0.0;
  int t = 0;
  for (; t + 2 <= trips; t += 2, c += 2 * G) {
    norm_load(table, c + G, chunks, b, lb);
    s += norm_sum(a, la);
    norm_load(table, c + 2 * G, chunks, a, la);
    s += norm_sum(b, lb);
  }
  if (t < trips) s += norm_sum(a, la);
  const double total = block_sum(s, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = total;
}

// Total of the partial sums; also reports the norm.
__global__ __launch_bounds__(256) void grad_sqnorm_final_kernel(const double* __restrict__ partial,
                                                                int groups, double* sqnorm,
                                                                double* grad_norm) {
  __shared__ double red[4];
  double s = 0.0;
#pragma unroll 8
  for (int i = threadIdx.x; i < groups; i += 256) s += partial[i];
  const double total = block_sum(s, red);
  if (threadIdx.x == 0) {
    *sqnorm = total;
    if (grad_norm) *grad_norm = sqrt(total);
  }
}

// Elementwise step, one workgroup per chunk: sixteen 16-byte loads per thread (4 x g, p, m, v)
// issued before any arithmetic; loads past the chunk's end are clamped to its last float4 and
// their results not stored.
__global__ __launch_bounds__(256) void adamw_kernel(const OptChunk* __restrict__ table,
                                                    const OptScalars c, const double* sqnorm) {
  constexpr int kIt = kOptChunk / 1024;
  const OptChunk ch = table[blockIdx.x];
  const int64_t n = ch.len;
  f32x4 g[kIt], p[kIt], m[kIt], v[kIt];
#pragma unroll
  for (int i = 0; i < kIt; ++i) {
    const int64_t e = 4 * ((int64_t)threadIdx.x + 256 * i);
    const int64_t ec = e < n ? e : n - 4;
    g[i] = *as_global(reinterpret_cast<const f32x4*>(ch.g + ec));
    p[i] = *as_global(reinterpret_cast<const f32x4*>(ch.p + ec));
    m[i] = *as_global(reinterpret_cast<const f32x4*>(ch.m + ec));
    v[i] = *as_global(reinterpret_cast<const f32x4*>(ch.v + ec));
  }
  const double norm = sqrt(*sqnorm);
  const float clip = c.max_norm > 0.f ? (float)fmin(1.0, (double)c.max_norm / (norm + 1e-6)) : 1.f;
  const float b1 = c.beta1, b2 = c.beta2, ob1 = 1.f - c.beta1, ob2 = 1.f - c.beta2;
#pragma unroll
  for (int i = 0; i < kIt; ++i) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float gk = __fmul_rn(g[i][k], clip);
      m[i][k] = __fadd_rn(__fmul_rn(b1, m[i][k]), __fmul_rn(ob1, gk));
      v[i][k] = __fadd_rn(__fmul_rn(b2, v[i][k]), __fmul_rn(ob2, __fmul_rn(gk, gk)));
      const float denom = __fadd_rn(__fmul_rn(sqrtf(v[i][k]), c.inv_sqrt_bc2), c.eps);
      p[i][k] = __fsub_rn(__fmul_rn(p[i][k], c.decay), __fmul_rn(c.step_size, __fdiv_rn(m[i][k], denom)));
    }
  }
#pragma unroll
  for (int i = 0; i < kIt; ++i) {
    const int64_t e = 4 * ((int64_t)threadIdx.x + 256 * i);
    if (e >= n) continue;
    *as_global(reinterpret_cast<f32x4*>(ch.p + e)) = p[i];
    *as_global(reinterpret_cast<f32x4*>(ch.m + e)) = m[i];
    *as_global(reinterpret_cast<f32x4*>(ch.v + e)) = v[i];
    if (ch.pb)
      *as_global(reinterpret_cast<u32x2*>(ch.pb + e)) =
          u32x2{pack_bf16x2(p[i][0], p[i][1]), pack_bf16x2(p[i][2], p[i][3])};
  }
}

// ------------------------------------------------------------------------------------------
int64_t opt_chunk_count(int64_t count, const int64_t* numel) {
  int64_t chunks = 0;
  for (int64_t i = 0; i < count; ++i) chunks += (numel[i] + kOptChunk - 1) / kOptChunk;
  return chunks;
}

// Device memory of a plan, one allocation: [chunk table][partial sums of the norm][sqnorm].
struct OptPlanDev {
  OptChunk* table;
  double* partial;
  double* sqnorm;
};

static int64_t plan_groups(int64_t chunks) { return chunks < kOptNormGrid ? chunks : kOptNormGrid; }

static OptPlanDev plan_dev(void* mem, int64_t chunks) {
  char* b = static_cast<char*>(mem);
  const size_t table_bytes = (size_t)chunks * sizeof(OptChunk);
  OptPlanDev d;
  d.table = reinterpret_cast<OptChunk*>(b);
  d.partial = reinterpret_cast<double*>(b + table_bytes);
  d.sqnorm = reinterpret_cast<double*>(b + table_bytes + (size_t)plan_groups(chunks) * sizeof(double));
  return d;
}

hipError_t opt_plan_create(int64_t count, float* const* params, const float* const* grads,
                           float* const* exp_avg, float* const* exp_avg_sq,
                           uint16_t* const* params_bf16, const int64_t* numel, void** dev_mem,
                           int64_t* chunks_out) {
  const int64_t chunks = opt_chunk_count(count, numel);
  const size_t table_bytes = (size_t)chunks * sizeof(OptChunk);
  OptChunk* host = static_cast<OptChunk*>(malloc(table_bytes));
  if (!host) return hipErrorOutOfMemory;
  int64_t c = 0;
  for (int64_t i = 0; i < count; ++i) {
    for (int64_t off = 0; off < numel[i]; off += kOptChunk, ++c) {
      OptChunk& d = host[c];
      d.p = params[i] + off;
      d.g = grads[i] + off;
      d.m = exp_avg[i] + off;
      d.v = exp_avg_sq[i] + off;
      d.pb = (params_bf16 && params_bf16[i]) ? params_bf16[i] + off : nullptr;
      d.len = numel[i] - off < kOptChunk ? numel[i] - off : kOptChunk;
    }
  }
  void* mem = nullptr;
  hipError_t e = hipMalloc(&mem, table_bytes + (size_t)(plan_groups(chunks) + 1) * sizeof(double));
  if (e == hipSuccess) e = hipMemcpy(mem, host, table_bytes, hipMemcpyHostToDevice);
  free(host);
  if (e != hipSuccess) {
    if (mem) (void)hipFree(mem);
    return e;
  }
  *dev_mem = mem;
  *chunks_out = chunks;
  return hipSuccess;
}

hipError_t opt_plan_step(void* dev_mem, int64_t chunks, float lr, float beta1, float beta2, float eps,
                         float weight_decay, float max_norm, int64_t step, double* grad_norm,
                         hipStream_t stream) {
  const OptPlanDev d = plan_dev(dev_mem, chunks);
  const int groups = (int)plan_groups(chunks);
  hipLaunchKernelGGL(grad_sqnorm_partial_kernel, dim3((unsigned)groups), dim3(256), 0, stream,
                     (const OptChunk*)d.table, (int)chunks, d.partial);
  hipLaunchKernelGGL(grad_sqnorm_final_kernel, dim3(1), dim3(256), 0, stream, (const double*)d.partial,
                     groups, d.sqnorm, grad_norm);
  const double bc1 = 1.0 - pow((double)beta1, (double)step);
  const double bc2 = 1.0 - pow((double)beta2, (double)step);
  OptScalars c;
  c.beta1 = beta1;
  c.beta2 = beta2;
  c.eps = eps;
  c.decay = (float)(1.0 - (double)lr * (double)weight_decay);
  c.step_size = (float)((double)lr / bc1);
  c.inv_sqrt_bc2 = (float)(1.0 / sqrt(bc2));
  c.max_norm = max_norm;
  hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)chunks), dim3(256), 0, stream, (const OptChunk*)d.table,
                     c, (const double*)d.sqnorm);
  return hipGetLastError();
}

}  // namespace nf4
