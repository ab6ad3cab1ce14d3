// Host-side launchers of the NF4 kernels. Each enqueues work on `stream` and returns the launch
// status; none synchronises or allocates.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4 {

hipError_t launch_quantize(const float* w, int64_t numel, uint8_t* packed, float* absmax,
                           hipStream_t stream);
hipError_t launch_double_quant(const float* absmax, int64_t nblocks, uint8_t* scale_q,
                               float* scale_c2, hipStream_t stream);
hipError_t launch_dequant(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                          int64_t numel, uint16_t* out, hipStream_t stream);

// absmax != null: fp32 scales per block instead of scale_q / scale_c2. part: room for
// fwd_gemm_splits(M, N, K) x M x N fp32 partial sums, or null (then the launch does not split)
int fwd_gemm_splits(int64_t M, int64_t N, int64_t K);
hipError_t launch_fwd_gemm(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                           const float* absmax, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                           const float* u, const uint16_t* B, int r, float scale, uint16_t* y,
                           float* part, hipStream_t stream);
hipError_t launch_dx_gemm(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                          const float* absmax, int64_t N, int64_t K, const uint16_t* dy, int64_t M,
                          const float* v, const uint16_t* A, int r, float scale, uint16_t* dx,
                          hipStream_t stream);

// Adapter passes over one bf16 matrix (see lora.hip). Each writes partial results to `ws`
// (lora_pass_ws_floats floats) and reduces them in a fixed order.
struct LoraPassPlan {
  int mb;           // rows per block
  int mblocks;      // row blocks
  int64_t crange;   // columns per column range
  int cranges;      // column ranges
};
LoraPassPlan lora_pass_plan(int64_t M, int64_t C, int r);
size_t lora_pass_ws_floats(int64_t M, int64_t C, int r, bool down, bool grad);
// u = X A^T
hipError_t launch_lora_u(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A, int r,
                         float* ws, float* u, hipStream_t stream);
// v = dY B and dB = scale * dY^T u (+ dB if accumulate), in one pass over dY
hipError_t launch_lora_dy(const uint16_t* dY, int64_t M, int64_t N, const uint16_t* B, const float* u,
                          int r, float scale, int accumulate, float* ws, float* v, float* dB,
                          hipStream_t stream);
// dA = scale * v^T X (+ dA if accumulate)
hipError_t launch_lora_dx(const uint16_t* X, int64_t M, int64_t K, const float* v, int r, float scale,
                          int accumulate, float* ws, float* dA, hipStream_t stream);

// Skinny forward (M <= 16): split-K dequant-GEMV on MFMA with a deterministic reduction.
// `part` holds skinny_workspace_floats(M, N, K, r) floats; u_out receives u = x A^T [M x r].
bool skinny_eligible(int64_t M, int64_t N, int64_t K);
struct SkinnyPlan {
  int w_blocks, w_splits, w_sub;   // items: row blocks x splits of w_sub steps
  int narrow;                      // M <= 4: 64-row blocks, 2048-column steps; else 256 rows, 512
};
SkinnyPlan skinny_plan(int64_t M, int64_t N, int64_t K, int r);
size_t skinny_workspace_floats(int64_t M, int64_t N, int64_t K, int r);
// absmax (fp32 block scales, scale_q / scale_c2 unused) is taken at M <= 4 only
hipError_t launch_skinny_fwd(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                             const float* absmax, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                             const uint16_t* A, const uint16_t* B, int r, float scale, float* part,
                             float* u_out,
                             uint16_t* y, hipStream_t stream);

// Adapter merged into the dequantised base: out = bf16(W~ + s B A), [N x K].
hipError_t launch_merge(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2, int64_t N,
                        int64_t K, const uint16_t* A, const uint16_t* B, int r, float scale, uint16_t* out,
                        hipStream_t stream);

// Adapter update over a plan: a device table of 4096-value chunk descriptors of every tensor.
int64_t opt_chunk_count(int64_t count, const int64_t* numel);
// allocates the plan's device memory (hipMalloc) and uploads the table (hipMemcpy, blocking)
hipError_t opt_plan_create(int64_t count, float* const* params, const float* const* grads,
                           float* const* exp_avg, float* const* exp_avg_sq,
                           uint16_t* const* params_bf16, const int64_t* numel, void** dev_mem,
                           int64_t* chunks_out);
// global squared norm, then the clipped AdamW step: three kernels on `stream`
hipError_t opt_plan_step(void* dev_mem, int64_t chunks, float lr, float beta1, float beta2, float eps,
                         float weight_decay, float max_norm, int64_t step, double* grad_norm,
                         hipStream_t stream);

// Codebook (0 NF4, 1 FP4 E2M1, 2 INT4) and blocksize (16..4096, a power of two) variants; the
// dequantisation takes fp32 scales (absmax != null) or double-quantised ones (scale_q, scale_c2).
bool q4_codebook(int id, float out[16], int* count);
hipError_t launch_q4_quantize(const float* w, int64_t numel, int book, int blocksize, uint8_t* packed,
                              float* absmax, hipStream_t stream);
hipError_t launch_q4_dequant(const uint8_t* packed, const float* absmax, const uint8_t* scale_q,
                             const float* scale_c2, int64_t numel, int book, int blocksize, uint16_t* out,
                             hipStream_t stream);

}  // namespace nf4
