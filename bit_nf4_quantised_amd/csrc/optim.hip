// The adapter update of a training step (gfx950): global gradient-norm clipping, then AdamW.
//
// "QLoRA, explained", The algorithm, step by step / Minimal implementation: after the backward the
// adapter gradients are clipped by their global norm (0.3 in the paper) and AdamW (32-bit state)
// updates A and B only. AdamW with decoupled weight decay, for clipped gradient g at step t:
//   p <- p (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;
//   p <- p - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps)
// with master weights and moments in fp32, and an optional bf16 copy of the new weights for the
// next forward (round to nearest even).
//
// Elementwise and bound by HBM: per element 16 bytes read (p, g, m, v) and 14 written (p, m, v,
// bf16 p). The norm is a separate pass (it must be complete before any element is updated): each
// workgroup sums the squares of a fixed 4096-element chunk in double, a tree in a fixed order, and
// one workgroup adds the chunk sums in chunk order, so the result is bitwise reproducible.
// Tensor lists (at most kOptMaxTensors per call) travel by value in the kernel arguments; a
// workgroup finds its tensor from the prefix sums of the chunk counts.
#include "common.h"
#include "launch.h"

namespace nf4 {

constexpr int kOptChunk = 4096;     // elements per workgroup: 256 threads x 4 float4

struct OptList {
  int count;
  int first[kOptMaxTensors + 1];    // first workgroup of each tensor; first[count] = grid
  int64_t n[kOptMaxTensors];
  const float* g[kOptMaxTensors];
  float* p[kOptMaxTensors];
  float* m[kOptMaxTensors];
  float* v[kOptMaxTensors];
  uint16_t* pb[kOptMaxTensors];
};

struct OptScalars {
  float beta1, beta2, eps, decay;   // decay = 1 - lr * weight_decay
  float step_size, inv_sqrt_bc2;    // lr / (1 - b1^t), 1 / sqrt(1 - b2^t)
  float max_norm;                   // <= 0: no clipping
};

__device__ __forceinline__ int tensor_of(const OptList& L, int wg) {
  int t = 0;
  while (t + 1 < L.count && L.first[t + 1] <= wg) ++t;
  return t;
}

// fixed-order sum of 256 doubles in LDS (thread 0 receives it)
__device__ __forceinline__ double block_sum(double x, double* red) {
  red[threadIdx.x] = x;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  return red[0];
}

__global__ __launch_bounds__(256) void grad_sqnorm_partial_kernel(const OptList L, double* partial) {
  __shared__ double red[256];
  const int wg = blockIdx.x;
  const int t = tensor_of(L, wg);
  const int64_t base = (int64_t)(wg - L.first[t]) * kOptChunk;
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kOptChunk / 1024; ++i) {
    const int64_t e = base + 4 * ((int64_t)threadIdx.x + 256 * i);
    if (e < L.n[t]) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(L.g[t] + e);
#pragma unroll
      for (int k = 0; k < 4; ++k) s += (double)x[k] * (double)x[k];
    }
  }
  const double total = block_sum(s, red);
  if (threadIdx.x == 0) partial[wg] = total;
}

__global__ __launch_bounds__(256) void grad_sqnorm_final_kernel(const double* partial, int nparts,
                                                                double* sqnorm, int accumulate) {
  __shared__ double red[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < nparts; i += 256) s += partial[i];
  const double total = block_sum(s, red);
  if (threadIdx.x == 0) *sqnorm = accumulate ? *sqnorm + total : total;
}

__global__ __launch_bounds__(256) void adamw_kernel(const OptList L, const OptScalars c,
                                                    const double* sqnorm, float* grad_norm) {
  const int wg = blockIdx.x;
  const int t = tensor_of(L, wg);
  const int64_t base = (int64_t)(wg - L.first[t]) * kOptChunk;
  const double norm = sqrt(*sqnorm);
  const float clip = c.max_norm > 0.f ? (float)fmin(1.0, (double)c.max_norm / (norm + 1e-6)) : 1.f;
  if (wg == 0 && threadIdx.x == 0 && grad_norm) *grad_norm = (float)norm;
  const float b1 = c.beta1, b2 = c.beta2, ob1 = 1.f - c.beta1, ob2 = 1.f - c.beta2;
#pragma unroll
  for (int i = 0; i < kOptChunk / 1024; ++i) {
    const int64_t e = base + 4 * ((int64_t)threadIdx.x + 256 * i);
    if (e >= L.n[t]) continue;
    const f32x4 g = *reinterpret_cast<const f32x4*>(L.g[t] + e);
    f32x4 p = *reinterpret_cast<const f32x4*>(L.p[t] + e);
    f32x4 m = *reinterpret_cast<const f32x4*>(L.m[t] + e);
    f32x4 v = *reinterpret_cast<const f32x4*>(L.v[t] + e);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float gk = __fmul_rn(g[k], clip);
      m[k] = __fadd_rn(__fmul_rn(b1, m[k]), __fmul_rn(ob1, gk));
      v[k] = __fadd_rn(__fmul_rn(b2, v[k]), __fmul_rn(ob2, __fmul_rn(gk, gk)));
      const float denom = __fadd_rn(__fmul_rn(sqrtf(v[k]), c.inv_sqrt_bc2), c.eps);
      p[k] = __fsub_rn(__fmul_rn(p[k], c.decay), __fmul_rn(c.step_size, __fdiv_rn(m[k], denom)));
    }
    *reinterpret_cast<f32x4*>(L.p[t] + e) = p;
    *reinterpret_cast<f32x4*>(L.m[t] + e) = m;
    *reinterpret_cast<f32x4*>(L.v[t] + e) = v;
    if (L.pb[t])
      *reinterpret_cast<u32x2*>(L.pb[t] + e) = u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
  }
}

// ------------------------------------------------------------------------------------------
static int opt_grid(OptList& L, const int64_t* numel) {
  int wgs = 0;
  for (int i = 0; i < L.count; ++i) {
    L.first[i] = wgs;
    L.n[i] = numel[i];
    wgs += (int)((numel[i] + kOptChunk - 1) / kOptChunk);
  }
  L.first[L.count] = wgs;
  return wgs;
}

size_t opt_workspace_bytes(int count, const int64_t* numel) {
  int64_t wgs = 0;
  for (int i = 0; i < count; ++i) wgs += (numel[i] + kOptChunk - 1) / kOptChunk;
  return (size_t)wgs * sizeof(double);
}

hipError_t launch_grad_sqnorm(int count, const float* const* grads, const int64_t* numel, double* ws,
                              double* sqnorm, int accumulate, hipStream_t stream) {
  OptList L{};
  L.count = count;
  for (int i = 0; i < count; ++i) L.g[i] = grads[i];
  const int wgs = opt_grid(L, numel);
  hipLaunchKernelGGL(grad_sqnorm_partial_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, L, ws);
  hipLaunchKernelGGL(grad_sqnorm_final_kernel, dim3(1), dim3(256), 0, stream, (const double*)ws, wgs,
                     sqnorm, accumulate);
  return hipGetLastError();
}

hipError_t launch_adamw(int count, float* const* params, const float* const* grads, float* const* exp_avg,
                        float* const* exp_avg_sq, uint16_t* const* params_bf16, const int64_t* numel,
                        float lr, float beta1, float beta2, float eps, float weight_decay,
                        float max_norm, int64_t step, const double* sqnorm, float* grad_norm,
                        hipStream_t stream) {
  OptList L{};
  L.count = count;
  for (int i = 0; i < count; ++i) {
    L.g[i] = grads[i];
    L.p[i] = params[i];
    L.m[i] = exp_avg[i];
    L.v[i] = exp_avg_sq[i];
    L.pb[i] = params_bf16 ? params_bf16[i] : nullptr;
  }
  const int wgs = opt_grid(L, numel);
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
  hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, L, c, sqnorm, grad_norm);
  return hipGetLastError();
}

}  // namespace nf4
