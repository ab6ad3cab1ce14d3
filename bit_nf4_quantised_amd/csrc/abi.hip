// C ABI of the NF4 QLoRA linear layer: host-side validation and kernel sequencing.
// Declarations and the contract of every call are in include/qlora_nf4.h.
#include "../../include/qlora_nf4.h"

#include <math.h>
#include <string.h>

#include <new>

#include "common.h"
#include "launch.h"

namespace {

constexpr uint32_t kCodeBits[16] = {NF4_CODE_BITS};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_weight(const nf4_weight* W) {
  if (!W || !W->packed) return NF4_ERR_NULL;
  // exactly one kind of scales: double-quantised (scale_q and scale_c2) or fp32 (absmax)
  if (W->absmax ? (W->scale_q || W->scale_c2) : !(W->scale_q && W->scale_c2)) return NF4_ERR_NULL;
  if (W->N < 16 || W->K < 64 || W->N % 16 || W->K % 64) return NF4_ERR_SHAPE;
  if (W->N > (int64_t(1) << 31) || W->K > (int64_t(1) << 31)) return NF4_ERR_SHAPE;
  if (!aligned16(W->packed) || !aligned16(W->scale_q) || !aligned16(W->scale_c2) || !aligned16(W->absmax))
    return NF4_ERR_ALIGN;
  return NF4_OK;
}

int check_rank(int32_t r) { return (r >= 16 && r <= 128 && r % 16 == 0) ? NF4_OK : NF4_ERR_RANK; }

int from_hip(hipError_t e) { return e == hipSuccess ? NF4_OK : NF4_ERR_HIP; }

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

// Workspace layout (bytes, each region 256-aligned):
//   forward : [u (M*r fp32)] [partials: the skinny path's splits, or the GEMM's contraction ranges]
//   backward: [v (M*r fp32)] [partials of the pass over dY, then of the pass over X]
size_t fwd_part_floats(int64_t M, int64_t N, int64_t K, int r) {
  if (nf4::skinny_eligible(M, N, K)) return nf4::skinny_workspace_floats(M, N, K, r);
  const int ks = nf4::fwd_gemm_splits(M, N, K);
  return ks > 1 ? (size_t)ks * M * N : 0;
}
size_t fwd_ws(int64_t M, int64_t N, int64_t K, int r) {
  return align_up((size_t)M * r * 4) + align_up(fwd_part_floats(M, N, K, r) * 4);
}
size_t bwd_ws(int64_t M, int64_t N, int64_t K, int r) {
  size_t part = nf4::lora_pass_ws_floats(M, N, r, true, true);
  const size_t ga = nf4::lora_pass_ws_floats(M, K, r, false, true);
  if (ga > part) part = ga;
  return align_up((size_t)M * r * 4) + align_up(part * 4);
}

template <typename T>
int check_ptr_list(int64_t count, T* const* ptrs, uintptr_t align_mask, bool entries_may_be_null) {
  if (!ptrs) return NF4_ERR_NULL;
  for (int64_t i = 0; i < count; ++i) {
    if (!ptrs[i]) {
      if (entries_may_be_null) continue;
      return NF4_ERR_NULL;
    }
    if (reinterpret_cast<uintptr_t>(ptrs[i]) & align_mask) return NF4_ERR_ALIGN;
  }
  return NF4_OK;
}

}  // namespace

// the opaque plan of the adapter update: device memory holding the chunk table and scratch
struct qlora_adamw_plan {
  void* mem = nullptr;
  int64_t chunks = 0;
  int device = -1;
};

extern "C" {

const char* nf4_status_string(int status) {
  switch (status) {
    case NF4_OK: return "ok";
    case NF4_ERR_NULL: return "a required pointer is NULL";
    case NF4_ERR_SHAPE: return "a size violates the contract";
    case NF4_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case NF4_ERR_RANK: return "LoRA rank must be a multiple of 16 in 16..128";
    case NF4_ERR_WORKSPACE: return "workspace missing or too small";
    case NF4_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

void nf4_codebook(float out[16]) { memcpy(out, kCodeBits, sizeof(kCodeBits)); }

int64_t nf4_storage_bytes(int64_t numel) {
  if (numel < 0 || numel % 64) return -1;
  const int64_t nb = numel / 64;
  return numel / 2 + nb + 4 * ((nb + 255) / 256);
}

int nf4_quantize(const float* w, int64_t numel, uint8_t* packed, float* absmax, hipStream_t stream) {
  if (numel < 0 || numel % 64) return NF4_ERR_SHAPE;
  if (numel == 0) return NF4_OK;
  if (!w || !packed || !absmax) return NF4_ERR_NULL;
  if (!aligned16(w) || !aligned16(packed) || !aligned16(absmax)) return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_quantize(w, numel, packed, absmax, stream));
}

int nf4_double_quant(const float* absmax, int64_t nblocks, uint8_t* scale_q, float* scale_c2,
                     hipStream_t stream) {
  if (nblocks < 0) return NF4_ERR_SHAPE;
  if (nblocks == 0) return NF4_OK;
  if (!absmax || !scale_q || !scale_c2) return NF4_ERR_NULL;
  if (!aligned16(absmax) || !aligned16(scale_q) || !aligned16(scale_c2)) return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_double_quant(absmax, nblocks, scale_q, scale_c2, stream));
}

int nf4_dequant(const nf4_weight* W, uint16_t* out, hipStream_t stream) {
  int st = check_weight(W);
  if (st) return st;
  if (!out) return NF4_ERR_NULL;
  if (!aligned16(out)) return NF4_ERR_ALIGN;
  if (W->absmax)
    return from_hip(nf4::launch_q4_dequant(W->packed, W->absmax, nullptr, nullptr, W->N * W->K, 0, 64, out,
                                           stream));
  return from_hip(nf4::launch_dequant(W->packed, W->scale_q, W->scale_c2, W->N * W->K, out, stream));
}

int qlora_merge(const nf4_weight* W, const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                uint16_t* out, hipStream_t stream) {
  int st = check_weight(W);
  if (st) return st;
  if ((st = check_rank(r))) return st;
  if (W->absmax) return NF4_ERR_SHAPE;   // the merge reads double-quantised scales only
  if (!A || !B || !out) return NF4_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(out)) return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_merge(W->packed, W->scale_q, W->scale_c2, W->N, W->K, A, B, r, scale,
                                    out, stream));
}

size_t qlora_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r) {
  if (M < 0 || N < 16 || K < 64 || N % 16 || K % 64 || check_rank(r)) return 0;
  if (M == 0) return 0;
  size_t a = fwd_ws(M, N, K, r), b = bwd_ws(M, N, K, r);
  return a > b ? a : b;
}

int qlora_linear_fwd(const nf4_weight* W, const uint16_t* x, int64_t M, const uint16_t* A,
                     const uint16_t* B, int32_t r, float scale, uint16_t* y, float* u_out, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  int st = check_weight(W);
  if (st) return st;
  if (M < 0) return NF4_ERR_SHAPE;
  if ((st = check_rank(r))) return st;
  if (M == 0) return NF4_OK;
  if (!x || !A || !B || !y) return NF4_ERR_NULL;
  if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(y) ||
      (u_out && !aligned16(u_out)) || (ws && !aligned16(ws)))
    return NF4_ERR_ALIGN;
  const int64_t N = W->N, K = W->K;
  const size_t need = fwd_ws(M, N, K, r);
  if (!ws || ws_bytes < need) return NF4_ERR_WORKSPACE;
  float* u = u_out ? u_out : static_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)M * r * 4));
  if (nf4::skinny_eligible(M, N, K) && (!W->absmax || M <= 4)) {
    return from_hip(nf4::launch_skinny_fwd(W->packed, W->scale_q, W->scale_c2, W->absmax, N, K, x, M, A, B, r,
                                           scale, part, u, y, stream));
  }
  hipError_t e = nf4::launch_lora_u(x, M, K, A, r, part, u, stream);
  if (e != hipSuccess) return NF4_ERR_HIP;
  return from_hip(nf4::launch_fwd_gemm(W->packed, W->scale_q, W->scale_c2, W->absmax, N, K, x, M, u, B,
                                       r, scale, y, part, stream));
}

int qlora_linear_fwd_recompute(const nf4_weight* W, const uint16_t* x, int64_t M, const uint16_t* A,
                               const uint16_t* B, int32_t r, float scale, const float* u, uint16_t* y,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_weight(W);
  if (st) return st;
  if (M < 0) return NF4_ERR_SHAPE;
  if ((st = check_rank(r))) return st;
  if (M == 0) return NF4_OK;
  if (!x || !A || !B || !u || !y) return NF4_ERR_NULL;
  if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(u) || !aligned16(y) ||
      (ws && !aligned16(ws)))
    return NF4_ERR_ALIGN;
  const int64_t N = W->N, K = W->K;
  if (nf4::skinny_eligible(M, N, K) && (!W->absmax || M <= 4)) {
    // the skinny path forms u itself from the adapter rows; it needs the workspace
    const size_t need = fwd_ws(M, N, K, r);
    if (!ws || ws_bytes < need) return NF4_ERR_WORKSPACE;
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)M * r * 4));
    float* u_scratch = static_cast<float*>(ws);
    return from_hip(nf4::launch_skinny_fwd(W->packed, W->scale_q, W->scale_c2, W->absmax, N, K, x, M, A, B, r,
                                           scale, part, u_scratch, y, stream));
  }
  // with a workspace of the forward's size, the same launches as qlora_linear_fwd (and the same
  // output bit for bit); without one, the GEMM in one pass over the contraction
  float* gpart = nullptr;
  if (ws && ws_bytes >= fwd_ws(M, N, K, r) && fwd_part_floats(M, N, K, r) > 0)
    gpart = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)M * r * 4));
  return from_hip(nf4::launch_fwd_gemm(W->packed, W->scale_q, W->scale_c2, W->absmax, N, K, x, M, u, B,
                                       r, scale, y, gpart, stream));
}

int qlora_linear_bwd(const nf4_weight* W, const uint16_t* x, const uint16_t* dy, int64_t M,
                     const uint16_t* A, const uint16_t* B, int32_t r, float scale, const float* u,
                     uint16_t* dx, float* dA, float* dB, int accumulate, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  int st = check_weight(W);
  if (st) return st;
  if (M < 0) return NF4_ERR_SHAPE;
  if ((st = check_rank(r))) return st;
  if (M == 0) return NF4_OK;
  if (!x || !dy || !A || !B || !u || !dA || !dB) return NF4_ERR_NULL;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(A) || !aligned16(B) || !aligned16(u) ||
      (dx && !aligned16(dx)) || !aligned16(dA) || !aligned16(dB) || (ws && !aligned16(ws)))
    return NF4_ERR_ALIGN;
  const int64_t N = W->N, K = W->K;
  const size_t need = bwd_ws(M, N, K, r);
  if (!ws || ws_bytes < need) return NF4_ERR_WORKSPACE;
  float* v = static_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)M * r * 4));
  hipError_t e = nf4::launch_lora_dy(dy, M, N, B, u, r, scale, accumulate, part, v, dB, stream);
  if (e != hipSuccess) return NF4_ERR_HIP;
  if (dx) {
    e = nf4::launch_dx_gemm(W->packed, W->scale_q, W->scale_c2, W->absmax, N, K, dy, M, v, A, r, scale, dx,
                            stream);
    if (e != hipSuccess) return NF4_ERR_HIP;
  }
  return from_hip(nf4::launch_lora_dx(x, M, K, v, r, scale, accumulate, part, dA, stream));
}

int q4_codebook_values(int32_t codebook, float out[16]) {
  if (!out) return NF4_ERR_NULL;
  int count = 0;
  return nf4::q4_codebook(codebook, out, &count) ? count : -NF4_ERR_SHAPE;
}

static int check_q4(int64_t numel, int32_t codebook, int32_t blocksize) {
  float q[16];
  int count = 0;
  if (!nf4::q4_codebook(codebook, q, &count)) return NF4_ERR_SHAPE;
  if (blocksize < 16 || blocksize > 4096 || (blocksize & (blocksize - 1))) return NF4_ERR_SHAPE;
  if (numel < 0 || numel % 64 || numel % blocksize || numel > (int64_t(1) << 42)) return NF4_ERR_SHAPE;
  return NF4_OK;
}

int q4_quantize(const float* w, int64_t numel, int32_t codebook, int32_t blocksize, uint8_t* packed,
                float* absmax, hipStream_t stream) {
  int st = check_q4(numel, codebook, blocksize);
  if (st) return st;
  if (numel == 0) return NF4_OK;
  if (!w || !packed || !absmax) return NF4_ERR_NULL;
  if (!aligned16(w) || !aligned16(packed) || !aligned16(absmax)) return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_q4_quantize(w, numel, codebook, blocksize, packed, absmax, stream));
}

int q4_dequant(const uint8_t* packed, int64_t numel, int32_t codebook, int32_t blocksize, const float* absmax,
               const uint8_t* scale_q, const float* scale_c2, uint16_t* out, hipStream_t stream) {
  int st = check_q4(numel, codebook, blocksize);
  if (st) return st;
  if (numel == 0) return NF4_OK;
  if (!packed || !out) return NF4_ERR_NULL;
  const bool dq = scale_q || scale_c2;
  if (absmax ? dq : !(scale_q && scale_c2)) return NF4_ERR_NULL;   // exactly one kind of scales
  if (!aligned16(packed) || !aligned16(out) || (absmax && !aligned16(absmax)) ||
      (scale_q && !aligned16(scale_q)) || (scale_c2 && !aligned16(scale_c2)))
    return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_q4_dequant(packed, absmax, scale_q, scale_c2, numel, codebook, blocksize, out,
                                         stream));
}

int qlora_adamw_plan_create(int64_t count, float* const* params, const float* const* grads,
                            float* const* exp_avg, float* const* exp_avg_sq, uint16_t* const* params_bf16,
                            const int64_t* numel, qlora_adamw_plan** out) {
  if (!out) return NF4_ERR_NULL;
  *out = nullptr;
  if (count < 1 || count > (int64_t(1) << 31)) return NF4_ERR_SHAPE;
  if (!numel) return NF4_ERR_NULL;
  for (int64_t i = 0; i < count; ++i)
    if (numel[i] <= 0 || numel[i] % 4 || numel[i] > (int64_t(1) << 40)) return NF4_ERR_SHAPE;
  if (nf4::opt_chunk_count(count, numel) > (int64_t(1) << 30)) return NF4_ERR_SHAPE;
  int st;
  if ((st = check_ptr_list(count, params, 15, false)) || (st = check_ptr_list(count, grads, 15, false)) ||
      (st = check_ptr_list(count, exp_avg, 15, false)) || (st = check_ptr_list(count, exp_avg_sq, 15, false)))
    return st;
  if (params_bf16 && (st = check_ptr_list(count, params_bf16, 7, true))) return st;
  qlora_adamw_plan* plan = new (std::nothrow) qlora_adamw_plan;
  if (!plan) return NF4_ERR_HIP;
  if (hipGetDevice(&plan->device) != hipSuccess ||
      nf4::opt_plan_create(count, params, grads, exp_avg, exp_avg_sq, params_bf16, numel, &plan->mem,
                           &plan->chunks) != hipSuccess) {
    delete plan;
    return NF4_ERR_HIP;
  }
  *out = plan;
  return NF4_OK;
}

int qlora_adamw_plan_step(const qlora_adamw_plan* plan, const qlora_adamw_config* cfg, int64_t step,
                          double* grad_norm, hipStream_t stream) {
  if (!plan || !cfg) return NF4_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(grad_norm) & 7u) return NF4_ERR_ALIGN;
  if (step < 1) return NF4_ERR_SHAPE;
  const qlora_adamw_config& c = *cfg;
  if (!isfinite(c.lr) || c.lr < 0.f || !(c.beta1 >= 0.f && c.beta1 < 1.f) ||
      !(c.beta2 >= 0.f && c.beta2 < 1.f) || !(c.eps > 0.f) || !isfinite(c.eps) ||
      !(c.weight_decay >= 0.f) || !isfinite(c.weight_decay) || isnan(c.max_grad_norm) ||
      isinf(c.max_grad_norm))
    return NF4_ERR_SHAPE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->device) return NF4_ERR_HIP;
  return from_hip(nf4::opt_plan_step(plan->mem, plan->chunks, c.lr, c.beta1, c.beta2, c.eps,
                                     c.weight_decay, c.max_grad_norm, step, grad_norm, stream));
}

int qlora_adamw_plan_destroy(qlora_adamw_plan* plan) {
  if (!plan) return NF4_OK;
  const hipError_t e = hipFree(plan->mem);
  delete plan;
  return from_hip(e);
}

}  // extern "C"
