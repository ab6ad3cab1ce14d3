// Host-side launchers of the NF4 kernels. Each enqueues work on `stream` and returns the launch
// status; none synchronises or allocates.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4 {

struct Codes;   // common.h

hipError_t launch_quantize(const float* w, int64_t numel, uint8_t* packed, float* absmax,
                           hipStream_t stream);
hipError_t launch_quantize_bf16(const uint16_t* w, int64_t numel, uint8_t* packed, float* absmax,
                                hipStream_t stream);
hipError_t launch_double_quant(const float* absmax, int64_t nblocks, uint8_t* scale_q,
                               float* scale_c2, hipStream_t stream);
// up to kDqBatch weights' scales per launch, passed by value in the kernel arguments
constexpr int kDqBatch = 64;
struct DqBatch {
  const float* absmax[kDqBatch];
  uint8_t* scale_q[kDqBatch];
  float* scale_c2[kDqBatch];
  int64_t nblocks[kDqBatch];
  int64_t group_begin[kDqBatch + 1];   // prefix sums of ceil(nblocks / 256)
  int count;
};
hipError_t launch_double_quant_many(const DqBatch& b, hipStream_t stream);
hipError_t launch_dequant(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                          int64_t numel, uint16_t* out, hipStream_t stream);

// The values of codebook `book` (0 NF4, 1 FP4 E2M1, 2 INT4); false for an unknown codebook. The
// linear, few-token and merge kernels take them by value.
bool codes_of(int book, Codes& out);

// absmax != null: fp32 scales per block instead of scale_q / scale_c2. part: room for
// fwd_gemm_part_floats(M, N, K) (forward) or dx_gemm_part_floats(M, N, K) (dX) fp32 partial sums,
// or null (then no tile's contraction is split)
size_t fwd_gemm_part_floats(int64_t M, int64_t N, int64_t K);
size_t dx_gemm_part_floats(int64_t M, int64_t N, int64_t K);
hipError_t launch_fwd_gemm(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                           const float* absmax, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                           const float* u, const uint16_t* B, int r, float scale, uint16_t* y,
                           float* part, int book, hipStream_t stream);
// A grouped forward: several linears that share x (and K, r, scale, codebook and kind of scales),
// as one launch. Eligible when M > 128 and their 256-row tiles number at least 192.
struct FwdGroupItem {
  const uint8_t* packed;
  const uint8_t* scale_q;
  const float* scale_c2;
  const float* absmax;
  int64_t N;
  const float* u;        // u = x A^T of this linear [M x r]
  const uint16_t* B;     // [N x r]
  uint16_t* y;           // [M x N]
};
bool fwd_group_eligible(int count, const int64_t* N, int64_t M, int64_t K);
size_t fwd_group_part_floats(int count, const int64_t* N, int64_t M, int64_t K);
hipError_t launch_fwd_gemm_group(int count, const FwdGroupItem* items, int64_t K, const uint16_t* x, int64_t M,
                                 int r, float scale, float* part, int book, hipStream_t stream);
// A grouped dX: several linears that share x, each dX_i = dY_i W~_i + s v_i A_i into its own dx_i,
// as one launch (the same per-tile arithmetic as launch_dx_gemm without partial sums). Eligible when
// M > 128 and their 256-row tiles number at least 192.
struct DxGroupItem {
  const uint8_t* packed;
  const uint8_t* scale_q;
  const float* scale_c2;
  const float* absmax;
  int64_t N;
  const uint16_t* dy;    // [M x N]
  const float* v;        // v = dY B [M x r]
  const uint16_t* A;     // [r x K]
  uint16_t* dx;          // [M x K]
};
bool dx_group_eligible(int count, int64_t M, int64_t K);
hipError_t launch_dx_gemm_group(int count, const DxGroupItem* items, int64_t K, int64_t M, int r, float scale,
                                int book, hipStream_t stream);
hipError_t launch_dx_gemm(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                          const float* absmax, int64_t N, int64_t K, const uint16_t* dy, int64_t M,
                          const float* v, const uint16_t* A, int r, float scale, uint16_t* dx,
                          float* part, int book, hipStream_t stream);

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
// u = X A^T. Above rank 16 (lora_u_uses_pass) it takes lora_pass_ws_floats(M, K, r, true, false)
// floats of ws for partial sums; at rank 16 ws is not used.
bool lora_u_uses_pass(int r);
hipError_t launch_lora_u(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A, int r,
                         float* ws, float* u, hipStream_t stream);
// u_i = X A_i^T for `count` (<= 8) linears of rank 16 that share X, in one launch (each u_i as
// launch_lora_u forms it, bit for bit)
hipError_t launch_lora_u_group(const uint16_t* X, int64_t M, int64_t K, int count, const uint16_t* const* A,
                               float* const* u, hipStream_t stream);
// v = dY B and dB = scale * dY^T u (+ dB if accumulate), in one pass over dY
hipError_t launch_lora_dy(const uint16_t* dY, int64_t M, int64_t N, const uint16_t* B, const float* u,
                          int r, float scale, int accumulate, float* ws, float* v, float* dB,
                          hipStream_t stream);
// dA = scale * v^T X (+ dA if accumulate)
hipError_t launch_lora_dx(const uint16_t* X, int64_t M, int64_t K, const float* v, int r, float scale,
                          int accumulate, float* ws, float* dA, hipStream_t stream);
// The same for `count` linears at once, each result bit for bit as the one-linear call gives it.
// dY side (count <= 4): every linear's pass, then one launch of the ordered sums of all of them; ws
// holds lora_dy_group_ws_floats floats (each linear's partial sums in turn).
struct LoraDyItem {
  const uint16_t* dY;
  int64_t N;
  const uint16_t* B;
  const float* u;
  float* v;
  float* dB;
};
size_t lora_dy_group_ws_floats(int count, const int64_t* N, int64_t M, int r);
hipError_t launch_lora_dy_group(int count, const LoraDyItem* it, int64_t M, int r, float scale, int accumulate,
                                float* ws, hipStream_t stream);
// X side (count <= 4 linears sharing X): dA_i = scale * v_i^T X; ws holds lora_dx_group_ws_floats floats
size_t lora_dx_group_ws_floats(int count, int64_t M, int64_t K, int r);
hipError_t launch_lora_dx_group(int count, const uint16_t* X, int64_t M, int64_t K, const float* const* v, int r,
                                float scale, int accumulate, float* ws, float* const* dA, hipStream_t stream);

// Skinny forward (M <= 16): split-K dequant-GEMV on MFMA with a deterministic reduction.
// `part` holds skinny_workspace_floats(M, N, K, r) floats; u_out receives u = x A^T [M x r].
bool skinny_eligible(int64_t M, int64_t N, int64_t K);
struct SkinnyPlan {
  int w_blocks, w_splits, w_sub;   // items: row blocks x splits of w_sub steps
  int narrow;                      // M <= 4: 64-row blocks, 2048-column steps; else 256 rows, 512
};
SkinnyPlan skinny_plan(int64_t M, int64_t N, int64_t K, int r);
size_t skinny_workspace_floats(int64_t M, int64_t N, int64_t K, int r);
// absmax != null: fp32 block scales (scale_q / scale_c2 unused)
hipError_t launch_skinny_fwd(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2,
                             const float* absmax, int64_t N, int64_t K, const uint16_t* x, int64_t M,
                             const uint16_t* A, const uint16_t* B, int r, float scale, float* part,
                             float* u_out, uint16_t* y, int book, hipStream_t stream);

// Adapter merged into the dequantised base: out = bf16(W~ + s B A), [N x K].
hipError_t launch_merge(const uint8_t* packed, const uint8_t* scale_q, const float* scale_c2, int64_t N,
                        int64_t K, const uint16_t* A, const uint16_t* B, int r, float scale, uint16_t* out,
                        int book, hipStream_t stream);

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
