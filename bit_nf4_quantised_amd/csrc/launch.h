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

hipError_t launch_fwd_gemm(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                           int64_t N, int64_t K, const uint16_t* x, int64_t M, const float* u,
                           const uint16_t* B, int r, float scale, uint16_t* y, hipStream_t stream);
hipError_t launch_dx_gemm(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                          int64_t N, int64_t K, const uint16_t* dy, int64_t M, const float* v,
                          const uint16_t* A, int r, float scale, uint16_t* dx, hipStream_t stream);

// u = P Q^T-like down projections (see lora.hip); `part` holds lora_down_chunks(M, L) * M * r floats.
int lora_down_chunks(int64_t M, int64_t L);
hipError_t launch_lora_down(const uint16_t* P, int64_t M, int64_t L, const uint16_t* Q, bool q_is_lr,
                            int r, float* part, float* out, hipStream_t stream);
// Adapter gradient out = scale * Q^T P (fp32); `part` holds lora_grad_workspace_floats(M, C, r) floats.
size_t lora_grad_workspace_floats(int64_t M, int64_t C, int r);
hipError_t launch_lora_grad(const float* P, const uint16_t* Q, int64_t M, int64_t C, int r,
                            float scale, float* out, bool out_cr, int accumulate, float* part,
                            hipStream_t stream);

// Skinny forward (M <= 16): split-K dequant-GEMV on MFMA with a deterministic reduction.
// `part` holds skinny_workspace_floats(M, N, K, r) floats; u_out receives u = x A^T [M x r].
bool skinny_eligible(int64_t M);
void skinny_plan(int64_t N, int64_t K, int r, int* splits, int* sub_per_split, int* row_tiles);
size_t skinny_workspace_floats(int64_t M, int64_t N, int64_t K, int r);
hipError_t launch_skinny_fwd(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                             int64_t N, int64_t K, const uint16_t* x, int64_t M, const uint16_t* A,
                             const uint16_t* B, int r, float scale, float* part, float* u_out,
                             uint16_t* y, hipStream_t stream);

}  // namespace nf4
