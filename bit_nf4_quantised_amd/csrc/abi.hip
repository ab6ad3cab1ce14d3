// C ABI of the NF4 QLoRA linear layer: host-side validation and kernel sequencing.
// Declarations and the contract of every call are in include/qlora_nf4.h.
#include "../../include/qlora_nf4.h"

#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>

#include "common.h"
#include "launch.h"

// The forward's workspace for callers that cannot allocate: 64 MiB of device memory that each GPU
// the library runs on holds until the process ends. Its name is only a host-side stand-in; host
// code reaches it through the address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr uint32_t kCodeBits[16] = {NF4_CODE_BITS};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_weight(const nf4_weight* W) {
  if (!W || !W->packed) return NF4_ERR_NULL;
  // exactly one kind of scales: double-quantised (scale_q and scale_c2) or fp32 (absmax)
  if (W->absmax ? (W->scale_q || W->scale_c2) : !(W->scale_q && W->scale_c2)) return NF4_ERR_NULL;
  if (W->N < 16 || W->K < 64 || W->N % 16 || W->K % 64) return NF4_ERR_SHAPE;
  if (W->N > (int64_t(1) << 31) || W->K > (int64_t(1) << 31)) return NF4_ERR_SHAPE;
  if (W->codebook < Q4_CODEBOOK_NF4 || W->codebook > Q4_CODEBOOK_INT4) return NF4_ERR_SHAPE;
  if (!aligned16(W->packed) || !aligned16(W->scale_q) || !aligned16(W->scale_c2) || !aligned16(W->absmax))
    return NF4_ERR_ALIGN;
  return NF4_OK;
}

int check_rank(int32_t r) { return (r >= 16 && r <= 128 && r % 16 == 0) ? NF4_OK : NF4_ERR_RANK; }

// Sizes the linear calls' kernels can address. Their buffer records and offsets are 32-bit: the
// backward's packed-weight record spans up to N*K/2 bytes, an activation tile up to 256 rows of a
// matrix with N or K bf16 columns (512 * max(N, K) bytes), each below 2^31; a launch counts its
// workgroups, ceil(M / 64) * ceil(max(N, K) / 128), in 32 bits.
bool linear_shape_ok(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || M >= (int64_t(1) << 31)) return false;
  if (N >= (int64_t(1) << 22) || K >= (int64_t(1) << 22)) return false;
  if (N * K >= (int64_t(1) << 32)) return false;
  const int64_t mx = N > K ? N : K;
  return ((M + 63) / 64) * ((mx + 127) / 128) < (int64_t(1) << 31);
}

int from_hip(hipError_t e) { return e == hipSuccess ? NF4_OK : NF4_ERR_HIP; }

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

// Workspace layout (bytes, each region 256-aligned):
//   forward : [u (M*r fp32)] [partials: the skinny path's splits, or (in turn) those of u above rank
//             16 and the GEMM's contraction ranges]
//   backward: [v (M*r fp32)] [partials of the pass over dY, then of the dX GEMM's tail, then of the
//             pass over X (each launch's partials are consumed before the next one writes)]
size_t fwd_part_floats(int64_t M, int64_t N, int64_t K, int r) {
  // the split GEMM's partial sums, after the partial sums of u (the two launches run in turn)
  const size_t gemm = nf4::fwd_gemm_part_floats(M, N, K);
  const size_t lu = nf4::lora_u_uses_pass(r) ? nf4::lora_pass_ws_floats(M, K, r, true, false) : 0;
  // few tokens (either kind of scales): the skinny path's splits
  if (nf4::skinny_eligible(M, N, K)) return nf4::skinny_workspace_floats(M, N, K, r);
  return gemm > lu ? gemm : lu;
}
size_t fwd_ws(int64_t M, int64_t N, int64_t K, int r) {
  return align_up((size_t)M * r * 4) + align_up(fwd_part_floats(M, N, K, r) * 4);
}
size_t bwd_ws(int64_t M, int64_t N, int64_t K, int r) {
  size_t part = nf4::lora_pass_ws_floats(M, N, r, true, true);
  const size_t ga = nf4::lora_pass_ws_floats(M, K, r, false, true);
  const size_t gx = nf4::dx_gemm_part_floats(M, N, K);
  if (ga > part) part = ga;
  if (gx > part) part = gx;
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

// ---- the forward's workspace for callers that cannot allocate (qlora_linear_fwd_noalloc): the
// file-scope array `scratch` below. The device address comes from hipGetSymbolAddress, looked up
// once per device with that device current, and every use goes through it.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NF4_ERR_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return NF4_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return NF4_OK;
}

// Argument checks of the forward, shared by qlora_linear_fwd and qlora_linear_fwd_noalloc.
int check_fwd(const nf4_weight* W, const uint16_t* x, int64_t M, const uint16_t* A, const uint16_t* B,
              int32_t r, const uint16_t* y, const float* u_out) {
  int st = check_weight(W);
  if (st) return st;
  if (!linear_shape_ok(M, W->N, W->K)) return NF4_ERR_SHAPE;
  if ((st = check_rank(r))) return st;
  if (M == 0) return NF4_OK;
  if (!x || !A || !B || !y) return NF4_ERR_NULL;
  if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(y) || (u_out && !aligned16(u_out)))
    return NF4_ERR_ALIGN;
  return NF4_OK;
}

// The forward's launches with u and the partial sums (fwd_part_floats(M, N, K, r)) placed.
int run_fwd_at(const nf4_weight* W, const uint16_t* x, int64_t M, const uint16_t* A, const uint16_t* B,
               int32_t r, float scale, uint16_t* y, float* u, float* part, hipStream_t stream) {
  const int64_t N = W->N, K = W->K;
  if (nf4::skinny_eligible(M, N, K)) {
    return from_hip(nf4::launch_skinny_fwd(W->packed, W->scale_q, W->scale_c2, W->absmax, N, K, x, M, A, B, r,
                                           scale, part, u, y, W->codebook, stream));
  }
  hipError_t e = nf4::launch_lora_u(x, M, K, A, r, part, u, stream);
  if (e != hipSuccess) return NF4_ERR_HIP;
  return from_hip(nf4::launch_fwd_gemm(W->packed, W->scale_q, W->scale_c2, W->absmax, N, K, x, M, u, B,
                                       r, scale, y, part, W->codebook, stream));
}

// The forward's launches once the arguments are checked and ws holds fwd_ws(M, N, K, r) bytes.
int run_fwd(const nf4_weight* W, const uint16_t* x, int64_t M, const uint16_t* A, const uint16_t* B,
            int32_t r, float scale, uint16_t* y, float* u_out, void* ws, hipStream_t stream) {
  float* u = u_out ? u_out : static_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)M * r * 4));
  return run_fwd_at(W, x, M, A, B, r, scale, y, u, part, stream);
}

// Workspace of a grouped forward: [u of each linear (M*r fp32 each)] [partial sums: the largest of
// the group launch's tail and of each linear's own forward (u's partial sums above rank 16, the
// few-token path, or the linear alone when the group is not eligible)].
size_t fwd_group_ws(int count, const int64_t* N, int64_t M, int64_t K, int r) {
  size_t part = nf4::fwd_group_part_floats(count, N, M, K);
  for (int i = 0; i < count; ++i) {
    const size_t f = fwd_part_floats(M, N[i], K, r);
    if (f > part) part = f;
  }
  return (size_t)count * align_up((size_t)M * r * 4) + align_up(part * 4);
}

// Workspace of a grouped backward: [v of each linear (M*r fp32 each)] [partial sums: the largest of
// the passes over every dY, of a dX launch of one linear and of the passes over X].
size_t bwd_group_ws(int count, const int64_t* N, int64_t M, int64_t K, int r) {
  size_t part = nf4::lora_dy_group_ws_floats(count, N, M, r);
  const size_t ga = nf4::lora_dx_group_ws_floats(count, M, K, r);
  if (ga > part) part = ga;
  for (int i = 0; i < count; ++i) {
    const size_t x = nf4::dx_gemm_part_floats(M, N[i], K);
    if (x > part) part = x;
  }
  return (size_t)count * align_up((size_t)M * r * 4) + align_up(part * 4);
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

int nf4_quantize_bf16(const uint16_t* w, int64_t numel, uint8_t* packed, float* absmax, hipStream_t stream) {
  if (numel < 0 || numel % 64) return NF4_ERR_SHAPE;
  if (numel == 0) return NF4_OK;
  if (!w || !packed || !absmax) return NF4_ERR_NULL;
  if (!aligned16(w) || !aligned16(packed) || !aligned16(absmax)) return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_quantize_bf16(w, numel, packed, absmax, stream));
}

int nf4_double_quant(const float* absmax, int64_t nblocks, uint8_t* scale_q, float* scale_c2,
                     hipStream_t stream) {
  if (nblocks < 0) return NF4_ERR_SHAPE;
  if (nblocks == 0) return NF4_OK;
  if (!absmax || !scale_q || !scale_c2) return NF4_ERR_NULL;
  if (!aligned16(absmax) || !aligned16(scale_q) || !aligned16(scale_c2)) return NF4_ERR_ALIGN;
  return from_hip(nf4::launch_double_quant(absmax, nblocks, scale_q, scale_c2, stream));
}

int nf4_double_quant_many(int64_t count, const float* const* absmax, const int64_t* nblocks,
                          uint8_t* const* scale_q, float* const* scale_c2, hipStream_t stream) {
  if (count < 0 || count > (int64_t(1) << 31)) return NF4_ERR_SHAPE;
  if (count == 0) return NF4_OK;
  if (!absmax || !nblocks || !scale_q || !scale_c2) return NF4_ERR_NULL;
  for (int64_t i = 0; i < count; ++i) {
    if (nblocks[i] < 0 || nblocks[i] > (int64_t(1) << 40)) return NF4_ERR_SHAPE;
    if (nblocks[i] == 0) continue;
    if (!absmax[i] || !scale_q[i] || !scale_c2[i]) return NF4_ERR_NULL;
    if (!aligned16(absmax[i]) || !aligned16(scale_q[i]) || !aligned16(scale_c2[i])) return NF4_ERR_ALIGN;
  }
  for (int64_t i0 = 0; i0 < count; i0 += nf4::kDqBatch) {
    nf4::DqBatch b{};
    int n = 0;
    b.group_begin[0] = 0;
    for (int64_t i = i0; i < count && i < i0 + nf4::kDqBatch; ++i) {
      if (nblocks[i] == 0) continue;
      b.absmax[n] = absmax[i];
      b.scale_q[n] = scale_q[i];
      b.scale_c2[n] = scale_c2[i];
      b.nblocks[n] = nblocks[i];
      b.group_begin[n + 1] = b.group_begin[n] + (nblocks[i] + nf4::kGroup - 1) / nf4::kGroup;
      ++n;
    }
    b.count = n;
    if (n == 0) continue;
    if (b.group_begin[n] * 64 >= (int64_t(1) << 32)) return NF4_ERR_SHAPE;   // threads of one launch
    const int st = from_hip(nf4::launch_double_quant_many(b, stream));
    if (st) return st;
  }
  return NF4_OK;
}

int nf4_dequant(const nf4_weight* W, uint16_t* out, hipStream_t stream) {
  int st = check_weight(W);
  if (st) return st;
  if (!out) return NF4_ERR_NULL;
  if (!aligned16(out)) return NF4_ERR_ALIGN;
  if (W->absmax || W->codebook != Q4_CODEBOOK_NF4)
    return from_hip(nf4::launch_q4_dequant(W->packed, W->absmax, W->scale_q, W->scale_c2, W->N * W->K,
                                           W->codebook, 64, out, stream));
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
                                    out, W->codebook, stream));
}

size_t qlora_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r) {
  if (M < 0 || N < 16 || K < 64 || N % 16 || K % 64 || check_rank(r)) return 0;
  if (!linear_shape_ok(M, N, K)) return 0;
  if (M == 0) return 0;
  size_t a = fwd_ws(M, N, K, r), b = bwd_ws(M, N, K, r);
  return a > b ? a : b;
}

int qlora_linear_fwd(const nf4_weight* W, const uint16_t* x, int64_t M, const uint16_t* A,
                     const uint16_t* B, int32_t r, float scale, uint16_t* y, float* u_out, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  int st = check_fwd(W, x, M, A, B, r, y, u_out);
  if (st || M == 0) return st;
  if (ws && !aligned16(ws)) return NF4_ERR_ALIGN;
  if (!ws || ws_bytes < fwd_ws(M, W->N, W->K, r)) return NF4_ERR_WORKSPACE;
  return run_fwd(W, x, M, A, B, r, scale, y, u_out, ws, stream);
}

}  // extern "C"

namespace {

// The grouped forward; with `recompute`, u_i is given (u_in) and only the GEMMs run, as in
// qlora_linear_fwd_recompute.
int run_fwd_group(int32_t count, const nf4_weight* const* W, const uint16_t* x, int64_t M, const uint16_t* const* A,
                  const uint16_t* const* B, int32_t r, float scale, uint16_t* const* y, float* const* u_io,
                  bool recompute, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (count < 1 || count > 4) return NF4_ERR_SHAPE;
  if (!W || !A || !B || !y || (recompute && !u_io)) return NF4_ERR_NULL;
  int64_t N[4];
  for (int i = 0; i < count; ++i) {
    const int st = check_fwd(W[i], x, M, A[i], B[i], r, y[i], u_io ? u_io[i] : nullptr);
    if (st) return st;
    if (W[i]->K != W[0]->K || W[i]->codebook != W[0]->codebook || (W[i]->absmax == nullptr) != (W[0]->absmax == nullptr))
      return NF4_ERR_SHAPE;
    if (recompute && M > 0 && !u_io[i]) return NF4_ERR_NULL;
    N[i] = W[i]->N;
  }
  if (M == 0) return NF4_OK;
  const int64_t K = W[0]->K;
  if (ws && !aligned16(ws)) return NF4_ERR_ALIGN;
  if (!ws || ws_bytes < fwd_group_ws(count, N, M, K, r)) return NF4_ERR_WORKSPACE;
  const size_t uslot = align_up((size_t)M * r * 4);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + count * uslot);
  float* u[4];
  for (int i = 0; i < count; ++i)
    u[i] = u_io && u_io[i] ? u_io[i] : reinterpret_cast<float*>(static_cast<char*>(ws) + i * uslot);
  if (!nf4::fwd_group_eligible(count, N, M, K)) {
    for (int i = 0; i < count; ++i) {
      // linear by linear, as qlora_linear_fwd (or its recompute) would run each; the workspace
      // holds one linear's [u][partial sums] at its start
      const int st = recompute
          ? qlora_linear_fwd_recompute(W[i], x, M, A[i], B[i], r, scale, u[i], y[i], ws, ws_bytes, stream)
          : run_fwd_at(W[i], x, M, A[i], B[i], r, scale, y[i], u[i], part, stream);
      if (st) return st;
    }
    return NF4_OK;
  }
  nf4::FwdGroupItem it[4];
  if (!recompute && !nf4::lora_u_uses_pass(r)) {
    // rank 16: every u_i in one pass over x
    if (nf4::launch_lora_u_group(x, M, K, count, A, u, stream) != hipSuccess) return NF4_ERR_HIP;
  }
  for (int i = 0; i < count; ++i) {
    if (!recompute && nf4::lora_u_uses_pass(r) && nf4::launch_lora_u(x, M, K, A[i], r, part, u[i], stream) != hipSuccess)
      return NF4_ERR_HIP;
    it[i] = nf4::FwdGroupItem{W[i]->packed, W[i]->scale_q, W[i]->scale_c2, W[i]->absmax, N[i], u[i], B[i], y[i]};
  }
  return from_hip(nf4::launch_fwd_gemm_group(count, it, K, x, M, r, scale, part, W[0]->codebook, stream));
}

}  // namespace

extern "C" {

int qlora_linear_fwd_group(int32_t count, const nf4_weight* const* W, const uint16_t* x, int64_t M,
                           const uint16_t* const* A, const uint16_t* const* B, int32_t r, float scale,
                           uint16_t* const* y, float* const* u_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return run_fwd_group(count, W, x, M, A, B, r, scale, y, u_out, false, ws, ws_bytes, stream);
}

int qlora_linear_fwd_recompute_group(int32_t count, const nf4_weight* const* W, const uint16_t* x, int64_t M,
                                     const uint16_t* const* A, const uint16_t* const* B, int32_t r, float scale,
                                     float* const* u, uint16_t* const* y, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  return run_fwd_group(count, W, x, M, A, B, r, scale, y, u, true, ws, ws_bytes, stream);
}

size_t qlora_workspace_bytes_group(int32_t count, const int64_t* N, int64_t M, int64_t K, int32_t r) {
  if (count < 1 || count > 4 || !N || M < 0 || K < 64 || K % 64 || check_rank(r)) return 0;
  for (int i = 0; i < count; ++i)
    if (N[i] < 16 || N[i] % 16 || !linear_shape_ok(M, N[i], K)) return 0;
  if (M == 0) return 0;
  const size_t f = fwd_group_ws(count, N, M, K, r), b = bwd_group_ws(count, N, M, K, r);
  return f > b ? f : b;
}

int qlora_linear_bwd_group(int32_t count, const nf4_weight* const* W, const uint16_t* x, const uint16_t* const* dy,
                           int64_t M, const uint16_t* const* A, const uint16_t* const* B, int32_t r, float scale,
                           const float* const* u, uint16_t* const* dx, float* const* dA, float* const* dB,
                           int accumulate, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (count < 1 || count > 4) return NF4_ERR_SHAPE;
  if (!W || !dy || !A || !B || !u || !dA || !dB) return NF4_ERR_NULL;
  int64_t N[4];
  int st;
  for (int i = 0; i < count; ++i) {
    if ((st = check_weight(W[i]))) return st;
    if (!linear_shape_ok(M, W[i]->N, W[i]->K)) return NF4_ERR_SHAPE;
    if (W[i]->K != W[0]->K || W[i]->codebook != W[0]->codebook || (W[i]->absmax == nullptr) != (W[0]->absmax == nullptr))
      return NF4_ERR_SHAPE;
    N[i] = W[i]->N;
  }
  if ((st = check_rank(r))) return st;
  if (M == 0) return NF4_OK;
  if (!x || !aligned16(x) || (ws && !aligned16(ws))) return !x ? NF4_ERR_NULL : NF4_ERR_ALIGN;
  for (int i = 0; i < count; ++i) {
    if (!dy[i] || !A[i] || !B[i] || !u[i] || !dA[i] || !dB[i] || (dx && !dx[i])) return NF4_ERR_NULL;
    if (!aligned16(dy[i]) || !aligned16(A[i]) || !aligned16(B[i]) || !aligned16(u[i]) || !aligned16(dA[i]) ||
        !aligned16(dB[i]) || (dx && !aligned16(dx[i])))
      return NF4_ERR_ALIGN;
  }
  const int64_t K = W[0]->K;
  if (!ws || ws_bytes < bwd_group_ws(count, N, M, K, r)) return NF4_ERR_WORKSPACE;
  const size_t vslot = align_up((size_t)M * r * 4);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + count * vslot);
  float* v[4];
  nf4::LoraDyItem dyi[4];
  for (int i = 0; i < count; ++i) {
    v[i] = reinterpret_cast<float*>(static_cast<char*>(ws) + i * vslot);
    dyi[i] = nf4::LoraDyItem{dy[i], N[i], B[i], u[i], v[i], dB[i]};
  }
  if (nf4::launch_lora_dy_group(count, dyi, M, r, scale, accumulate, part, stream) != hipSuccess) return NF4_ERR_HIP;
  if (dx) {
    if (nf4::dx_group_eligible(count, M, K)) {
      // the longest contraction first, so that every XCD gets its share of each weight's tiles in
      // that order and ends with the short ones
      int order[4] = {0, 1, 2, 3};
      for (int a = 0; a < count; ++a)
        for (int b = a + 1; b < count; ++b)
          if (N[order[b]] > N[order[a]]) {
            const int t = order[a];
            order[a] = order[b];
            order[b] = t;
          }
      nf4::DxGroupItem it[4];
      for (int k = 0; k < count; ++k) {
        const int i = order[k];
        it[k] = nf4::DxGroupItem{W[i]->packed, W[i]->scale_q, W[i]->scale_c2, W[i]->absmax, N[i], dy[i], v[i], A[i], dx[i]};
      }
      if (nf4::launch_dx_gemm_group(count, it, K, M, r, scale, W[0]->codebook, stream) != hipSuccess) return NF4_ERR_HIP;
    } else {
      for (int i = 0; i < count; ++i)
        if (nf4::launch_dx_gemm(W[i]->packed, W[i]->scale_q, W[i]->scale_c2, W[i]->absmax, N[i], K, dy[i], M, v[i], A[i],
                                r, scale, dx[i], part, W[i]->codebook, stream) != hipSuccess)
          return NF4_ERR_HIP;
    }
  }
  return nf4::launch_lora_dx_group(count, x, M, K, v, r, scale, accumulate, part, dA, stream) == hipSuccess
             ? NF4_OK
             : NF4_ERR_HIP;
}

int qlora_linear_fwd_noalloc(const nf4_weight* W, const uint16_t* x, int64_t M, const uint16_t* A,
                             const uint16_t* B, int32_t r, float scale, uint16_t* y, float* u_out,
                             hipStream_t stream) {
  int st = check_fwd(W, x, M, A, B, r, y, u_out);
  if (st || M == 0) return st;
  if (fwd_ws(M, W->N, W->K, r) > kScratchBytes) return NF4_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws))) return st;
  return run_fwd(W, x, M, A, B, r, scale, y, u_out, ws, stream);
}

int qlora_linear_fwd_recompute(const nf4_weight* W, const uint16_t* x, int64_t M, const uint16_t* A,
                               const uint16_t* B, int32_t r, float scale, const float* u, uint16_t* y,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_weight(W);
  if (st) return st;
  if (!linear_shape_ok(M, W->N, W->K)) return NF4_ERR_SHAPE;
  if ((st = check_rank(r))) return st;
  if (M == 0) return NF4_OK;
  if (!x || !A || !B || !u || !y) return NF4_ERR_NULL;
  if (!aligned16(x) || !aligned16(A) || !aligned16(B) || !aligned16(u) || !aligned16(y) ||
      (ws && !aligned16(ws)))
    return NF4_ERR_ALIGN;
  const int64_t N = W->N, K = W->K;
  if (nf4::skinny_eligible(M, N, K)) {
    // the skinny path forms u itself from the adapter rows; it needs the workspace
    const size_t need = fwd_ws(M, N, K, r);
    if (!ws || ws_bytes < need) return NF4_ERR_WORKSPACE;
    float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)M * r * 4));
    float* u_scratch = static_cast<float*>(ws);
    return from_hip(nf4::launch_skinny_fwd(W->packed, W->scale_q, W->scale_c2, W->absmax, N, K, x, M, A, B, r,
                                           scale, part, u_scratch, y, W->codebook, stream));
  }
  // with a workspace of the forward's size, the same launches as qlora_linear_fwd (and the same
  // output bit for bit); without one, the GEMM in one pass over the contraction
  float* gpart = nullptr;
  if (ws && ws_bytes >= fwd_ws(M, N, K, r) && fwd_part_floats(M, N, K, r) > 0)
    gpart = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)M * r * 4));
  return from_hip(nf4::launch_fwd_gemm(W->packed, W->scale_q, W->scale_c2, W->absmax, N, K, x, M, u, B,
                                       r, scale, y, gpart, W->codebook, stream));
}

int qlora_linear_bwd(const nf4_weight* W, const uint16_t* x, const uint16_t* dy, int64_t M,
                     const uint16_t* A, const uint16_t* B, int32_t r, float scale, const float* u,
                     uint16_t* dx, float* dA, float* dB, int accumulate, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  int st = check_weight(W);
  if (st) return st;
  if (!linear_shape_ok(M, W->N, W->K)) return NF4_ERR_SHAPE;
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
                            part, W->codebook, stream);
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
