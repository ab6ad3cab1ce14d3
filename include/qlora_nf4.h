/* qlora_nf4.h - C ABI of the NF4-quantised QLoRA linear layer for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the method as stated on "QLoRA, explained" (pofe.ai):
 *   nf4_quantize      sections "Blockwise absmax quantisation" and "NormalFloat 4 (NF4)": a weight is
 *                     flattened row-major and cut into blocks of 64; a block keeps its absmax, and
 *                     every value becomes the position of its closest NF4 code (16 codes);
 *                     "Minimal implementation": two indices per byte.
 *   nf4_double_quant  section "Double quantisation": the block scales are quantised to 8-bit floats
 *                     in groups of 256 with one fp32 constant per group.
 *   nf4_dequant       section "The forward pass and gradients": first the 8-bit scales are restored
 *                     with the fp32 constants, then the indices with those scales, giving bf16.
 *   qlora_linear_fwd  section "The algorithm, step by step": y = x W~^T + s x A^T B^T
 *                     (qlora_linear_fwd_group: several linears that share x, as one launch).
 *   qlora_linear_bwd  section "The forward pass and gradients": dX = dY (W~ + s B A),
 *                     dA = s B^T G, dB = s G A^T with G = dY^T X; W gets no gradient.
 *   qlora_merge       section "Quality loss at merge time": the adapter merged into the
 *                     dequantised base, W~ + s B A, served in bf16; nf4_quantize_bf16 quantises
 *                     such a merged weight again.
 *   qlora_adamw_plan_*   sections "The algorithm, step by step" and "Minimal implementation":
 *                     global gradient-norm clipping, then AdamW over A and B.
 *   q4_*              sections "A toy run" and "Double quantisation": FP4 and INT4 codebooks,
 *                     blocksizes 16..4096, and fp32 scales without double quantisation.
 *
 * Data formats (all little-endian, row-major):
 *   W        N x K (out x in, like nn.Linear), K % 64 == 0, N % 16 == 0. Blocks of 64 run along K.
 *   packed   uint8[N*K/2]: byte j holds the code index of element 2j in its high nibble and of
 *            element 2j+1 in its low nibble. Codes are ascending; index 7 is the exact zero.
 *   scale_q  uint8[N*K/64]: OCP E4M3 code of c1[b] / c2[b / 256], the nearest E4M3 value in [0, 1]
 *            to the exact ratio, ties to the even code.
 *   scale_c2 float[ceil(N*K/64/256)]: c2[g] = max of the 256 block absmax values of group g.
 *   bf16     stored as uint16 bit patterns. Dequantised value: bf16_rne(fl32(q[idx] * c1')) with
 *            c1' = fl32(e4m3(scale_q) * c2); q is the NF4 codebook unless the weight names another.
 *   LoRA     A: bf16 r x K, B: bf16 N x r, scale s = lora_alpha / r; 16 <= r <= 128, r % 16 == 0.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers to caller-owned memory (except nf4_codebook's output, a host
 *     array), each 16-byte aligned. Apart from qlora_adamw_plan_create (which allocates the plan's
 *     device memory and blocks until its table is uploaded) and qlora_adamw_plan_destroy (which
 *     frees it), the library never allocates or frees device memory and never synchronises. Its
 *     only mutable global state is qlora_linear_fwd_noalloc's workspace (see there); every other
 *     call is thread-safe.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the default stream).
 *     The return value reports argument validation and launch status; faults inside kernels
 *     surface at the caller's next synchronisation.
 *   - Arguments are validated on the host before any HIP call; on error nothing is enqueued.
 *   - Inputs must be finite; NaN and Inf are outside the contract and are not checked.
 *   - Results are deterministic: every reduction runs in a fixed order without atomics.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NF4_OK = 0,
  NF4_ERR_NULL = 1,       /* a required pointer is NULL */
  NF4_ERR_SHAPE = 2,      /* a size violates the contract (see each call) */
  NF4_ERR_ALIGN = 3,      /* a pointer is not 16-byte aligned */
  NF4_ERR_RANK = 4,       /* r outside 16..128 or not a multiple of 16 */
  NF4_ERR_WORKSPACE = 5,  /* ws is NULL or smaller than qlora_workspace_bytes() */
  NF4_ERR_HIP = 6         /* the HIP runtime rejected a kernel launch */
} nf4_status;

/* The 4-bit codebooks ("QLoRA, explained", A toy run, which sets NF4 beside an INT4 grid of 15
 * levels k/7 and E2M1 FP4 rescaled to [-1, 1]). */
enum {
  Q4_CODEBOOK_NF4 = 0,    /* the 16 NF4 codes (nf4_codebook) */
  Q4_CODEBOOK_FP4 = 1,    /* E2M1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} / 6, both signs: 15 codes */
  Q4_CODEBOOK_INT4 = 2    /* k / 7 for k = -7..7: 15 codes */
};

/* A quantised weight W (N x K), device memory. Its block scales are either double quantised
 * (scale_q and scale_c2 set, absmax NULL: 4.127 bits per weight) or the fp32 absmax itself
 * (absmax set, scale_q and scale_c2 NULL: the 4.5-bit baseline without double quantisation,
 * "QLoRA, explained", Double quantisation). nf4_dequant, the linear calls (the few-token forward
 * path included) take either; with fp32 scales qlora_merge is not available (NF4_ERR_SHAPE).
 * codebook names the values the indices select: Q4_CODEBOOK_NF4 (0, what nf4_quantize writes),
 * or Q4_CODEBOOK_FP4 / Q4_CODEBOOK_INT4 for indices written by q4_quantize at blocksize 64 (their
 * indices must be below 15). Every call that takes an nf4_weight dequantises with it; any other
 * value is NF4_ERR_SHAPE. */
typedef struct {
  const uint8_t *packed;    /* [N*K/2]                 */
  const uint8_t *scale_q;   /* [N*K/64]                */
  const float *scale_c2;    /* [ceil(N*K/64/256)]      */
  int64_t N, K;
  const float *absmax;      /* [N*K/64] or NULL        */
  int32_t codebook;         /* Q4_CODEBOOK_*           */
} nf4_weight;

/* Blockwise absmax NF4 quantisation of a float32 array (any shape, flattened row-major).
 *   w       [numel] float32 input; numel % 64 == 0 (callers zero-pad), numel >= 0.
 *   packed  [numel/2] output, two indices per byte (see Data formats).
 *   absmax  [numel/64] output, exact float32 block maxima of |w| (first-level scales).
 * Nearest code: the exact real quotient w / absmax decides, ties to the lower index; a block
 * whose absmax is 0 stores index 7 everywhere.
 * Errors: NF4_ERR_NULL (w, packed or absmax NULL while numel > 0), NF4_ERR_SHAPE, NF4_ERR_ALIGN. */
int nf4_quantize(const float *w, int64_t numel, uint8_t *packed, float *absmax, hipStream_t stream);

/* nf4_quantize of a bf16 array (uint16 bit patterns), for re-quantising a merged weight: "QLoRA,
 * explained", section "Quality loss at merge time", names merging into W~ and quantising the
 * result again. Every bf16 value widens to float32 exactly, so packed and absmax are bit for bit
 * those of nf4_quantize on the widened array; the call reads 2 bytes per value instead of 4.
 *   w       [numel] bf16 input, 16-byte aligned; numel % 64 == 0.
 *   packed, absmax: as nf4_quantize.
 * Errors: as nf4_quantize. */
int nf4_quantize_bf16(const uint16_t *w, int64_t numel, uint8_t *packed, float *absmax, hipStream_t stream);

/* Double quantisation of block scales.
 *   absmax    [nblocks] float32 input (from nf4_quantize).
 *   scale_q   [nblocks] output E4M3 codes; scale_c2 [ceil(nblocks/256)] output group maxima
 *             (the last group may hold fewer than 256 scales; a group of zeros stores code 0).
 * Errors: NF4_ERR_NULL, NF4_ERR_SHAPE (nblocks < 0), NF4_ERR_ALIGN. */
int nf4_double_quant(const float *absmax, int64_t nblocks, uint8_t *scale_q, float *scale_c2,
                     hipStream_t stream);

/* nf4_double_quant over several weights: tensor i's absmax[i] (nblocks[i] scales) is encoded into
 * scale_q[i] and scale_c2[i] exactly as nf4_double_quant would, with up to 64 tensors per kernel
 * launch (their pointers travel in the kernel arguments; nothing is allocated). For a model's many
 * weights at load time, where a launch per weight would be bound by launch overhead.
 *   count      number of tensors (>= 0); absmax, nblocks, scale_q, scale_c2 are HOST arrays of
 *              `count` entries (device pointers and sizes); entries with nblocks[i] == 0 are skipped
 *              and may hold NULL pointers. Outputs must not overlap another tensor's inputs.
 * Errors: NF4_ERR_NULL, NF4_ERR_SHAPE (count or a size < 0), NF4_ERR_ALIGN, NF4_ERR_HIP; on an
 * argument error nothing is enqueued. */
int nf4_double_quant_many(int64_t count, const float *const *absmax, const int64_t *nblocks,
                          uint8_t *const *scale_q, float *const *scale_c2, hipStream_t stream);

/* Two-level dequantisation of W to bf16.
 *   out  [N*K] uint16 (bf16) output, row-major N x K; bit-exact with the formula in Data formats.
 * Errors: NF4_ERR_NULL, NF4_ERR_SHAPE (N % 16, K % 64, N < 16, K < 64), NF4_ERR_ALIGN. */
int nf4_dequant(const nf4_weight *W, uint16_t *out, hipStream_t stream);

/* Size limits of the three linear calls (their kernels address buffers with 32-bit offsets):
 * N < 2^22, K < 2^22, N*K < 2^32 and 0 <= M < 2^31, with ceil(M/64) * ceil(max(N, K)/128) < 2^31.
 * Larger sizes are refused with NF4_ERR_SHAPE (and qlora_workspace_bytes returns 0 for them);
 * nf4_quantize, nf4_dequant and qlora_merge index in 64 bits and take the weight whole.
 *
 * Forward of the adapted linear: y = x W~^T + s (x A^T) B^T, bf16 inputs, fp32 accumulation,
 * W~ dequantised on the fly (never written to memory).
 *   x      [M x K] bf16;  A [r x K] bf16;  B [N x r] bf16;  scale = s.
 *   y      [M x N] bf16 output.
 *   u_out  [M x r] float32 output u = x A^T (saved for qlora_linear_bwd), or NULL.
 *   ws     device workspace of at least qlora_workspace_bytes(M, N, K, r) bytes.
 * M == 0 is a no-op. Errors: NF4_ERR_NULL, NF4_ERR_SHAPE, NF4_ERR_ALIGN, NF4_ERR_RANK,
 * NF4_ERR_WORKSPACE, NF4_ERR_HIP. */
int qlora_linear_fwd(const nf4_weight *W, const uint16_t *x, int64_t M, const uint16_t *A,
                     const uint16_t *B, int32_t r, float scale, uint16_t *y, float *u_out, void *ws,
                     size_t ws_bytes, hipStream_t stream);

/* Forward of several adapted linears that share their input x, such as a layer's query, key and
 * value projections or its gate and up projections: y_i = x W~_i^T + s (x A_i^T) B_i^T for
 * i < count (1..4), each as in qlora_linear_fwd ("QLoRA, explained", The algorithm, step by step,
 * applied to every linear). All weights share K, the rank r, the scale, the codebook and the kind
 * of scales. Above 128 tokens, when the weights' 256-row tiles number at least 192 together, the
 * fused GEMMs run as one launch whose column tiles run over the weights in turn (fewer launches,
 * and small linears such as the key and value projections share the large one's efficiency);
 * otherwise each linear runs as qlora_linear_fwd runs it. The results are those of qlora_linear_fwd
 * up to the order in which the contraction is summed (within the forward's tolerance).
 *   W, A, B, y: HOST arrays of count entries, each as in qlora_linear_fwd.
 *   u_out: NULL, or a HOST array of count entries of which any may be NULL; u_i = x A_i^T goes there
 *          (for qlora_linear_bwd) or into the workspace.
 *   ws: at least qlora_workspace_bytes_group(count, N, M, K, r) bytes (N the weights' row counts).
 * Errors: as qlora_linear_fwd; NF4_ERR_SHAPE also for count outside 1..4 and for weights that
 * differ in K, codebook or kind of scales. */
int qlora_linear_fwd_group(int32_t count, const nf4_weight *const *W, const uint16_t *x, int64_t M,
                           const uint16_t *const *A, const uint16_t *const *B, int32_t r, float scale,
                           uint16_t *const *y, float *const *u_out, void *ws, size_t ws_bytes,
                           hipStream_t stream);
/* qlora_linear_fwd_group with every u_i = x A_i^T already known (u: HOST array of count device
 * pointers, all set), as qlora_linear_fwd_recompute is to qlora_linear_fwd: the GEMMs only, the
 * same launches as qlora_linear_fwd_group after its u (so y_i equal its output bit for bit).
 * Errors as qlora_linear_fwd_group. */
int qlora_linear_fwd_recompute_group(int32_t count, const nf4_weight *const *W, const uint16_t *x, int64_t M,
                                     const uint16_t *const *A, const uint16_t *const *B, int32_t r,
                                     float scale, float *const *u, uint16_t *const *y, void *ws,
                                     size_t ws_bytes, hipStream_t stream);
/* Backward of several adapted linears that share their input x (the group of
 * qlora_linear_fwd_group): for every i < count, as qlora_linear_bwd on linear i (dX_i, dA_i, dB_i
 * into its own outputs). Above 128 tokens, when the linears' 256-row dX tiles number at least 192
 * together, their dX GEMMs run as one launch (each dX_i is then computed exactly as a dX launch
 * without a split contraction computes it). The adapter work is batched the same way: the passes
 * over every dY_i as one launch, the passes over the shared x as one (a single pass for all dA_i
 * when the ranks add up to 64 or less), and their ordered sums in one launch each; every dA_i and
 * dB_i equals what qlora_linear_bwd returns for linear i, bit for bit.
 *   W, dy, A, B, u, dA, dB: HOST arrays of count entries, each as in qlora_linear_bwd.
 *   dx: NULL (no input gradient) or a HOST array of count device pointers, all set. A layer's
 *       gradient with respect to the shared x is the sum of the dX_i.
 *   ws: at least qlora_workspace_bytes_group(count, N, M, K, r) bytes.
 * Errors: as qlora_linear_bwd; NF4_ERR_SHAPE also for count outside 1..4 and for weights that
 * differ in K, codebook or kind of scales. */
int qlora_linear_bwd_group(int32_t count, const nf4_weight *const *W, const uint16_t *x,
                           const uint16_t *const *dy, int64_t M, const uint16_t *const *A,
                           const uint16_t *const *B, int32_t r, float scale, const float *const *u,
                           uint16_t *const *dx, float *const *dA, float *const *dB, int accumulate,
                           void *ws, size_t ws_bytes, hipStream_t stream);
/* Workspace bytes of qlora_linear_fwd_group, its recompute and qlora_linear_bwd_group for weights
 * of N[0..count-1] rows; 0 for sizes they refuse. N is a HOST array. */
size_t qlora_workspace_bytes_group(int32_t count, const int64_t *N, int64_t M, int64_t K, int32_t r);

/* qlora_linear_fwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same launches and the same outputs,
 * bit for bit, with the workspace taken from a 64 MiB array inside the library instead of `ws`.
 * Each GPU the library runs on holds its own copy of that array until the process ends; its
 * device address is looked up (hipGetSymbolAddress) on the first call on that device. The call
 * allocates nothing, and nothing in the array needs clearing: every launch overwrites what it
 * reads. All calls on one GPU share its array, so calls that overlap on one GPU (other streams or
 * threads without ordering between them) race.
 * Errors as qlora_linear_fwd; NF4_ERR_WORKSPACE when the forward's workspace for these sizes
 * (with u kept in it when u_out is NULL) exceeds 64 MiB; NF4_ERR_HIP when the array's address
 * cannot be obtained. */
int qlora_linear_fwd_noalloc(const nf4_weight *W, const uint16_t *x, int64_t M, const uint16_t *A,
                             const uint16_t *B, int32_t r, float scale, uint16_t *y, float *u_out,
                             hipStream_t stream);

/* Backward of the adapted linear given dY, with W~ dequantised again on the fly:
 *   dx = dY W~ + s (dY B) A          [M x K] bf16 output, or NULL to skip it;
 *   dA = s (dY B)^T x                [r x K] float32 output;
 *   dB = s dY^T u                    [N x r] float32 output, u = x A^T from qlora_linear_fwd.
 *   accumulate: 0 overwrites dA and dB, 1 adds into them. No gradient is produced for W.
 * M == 0 is a no-op. Errors as qlora_linear_fwd. */
int qlora_linear_bwd(const nf4_weight *W, const uint16_t *x, const uint16_t *dy, int64_t M,
                     const uint16_t *A, const uint16_t *B, int32_t r, float scale, const float *u,
                     uint16_t *dx, float *dA, float *dB, int accumulate, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/* Forward recompute with a known u = x A^T (as saved by qlora_linear_fwd): y = x W~^T + s u B^T.
 * "QLoRA, explained", section "Compute and memory cost": when gradient checkpointing recomputes the
 * forward, the weight is dequantised a third time per layer and step; the adapter down-projection
 * saved by the first forward is reused rather than recomputed. For M > 16 this runs the fused
 * dequantise + MFMA GEMM alone: one launch, or, when the output has too few tiles to fill the GPU
 * and ws holds qlora_workspace_bytes(M, N, K, r) bytes, the GEMM split over two contraction ranges
 * plus a launch that adds the two halves, exactly as qlora_linear_fwd does (so y equals its output
 * bit for bit). For M <= 16 it runs the skinny path (which forms u again from A) and needs ws.
 *   u   [M x r] float32 input.  y [M x N] bf16 output.  ws as qlora_linear_fwd (may be NULL if M > 16:
 *   then the GEMM is never split, same tolerance).
 * Errors as qlora_linear_fwd. */
int qlora_linear_fwd_recompute(const nf4_weight *W, const uint16_t *x, int64_t M, const uint16_t *A,
                               const uint16_t *B, int32_t r, float scale, const float *u, uint16_t *y,
                               void *ws, size_t ws_bytes, hipStream_t stream);

/* Adapter merged into the dequantised base weight, in bf16:
 *   out = bf16_rne(W~ + s (B A))      [N x K] bf16 output (uint16 bit patterns),
 * the exact value rounded once (nearest, ties to even), W~ exactly as nf4_dequant produces it.
 * "QLoRA, explained", section "Quality loss at merge time": training saw W~, never the original
 * weight, so adding the adapter to W~ preserves the trained model; the result is served in bf16
 * (re-quantising it, with nf4_quantize_bf16, rounds the update a second time).
 *   A [r x K] bf16;  B [N x r] bf16;  scale = s (used as given, in float).
 * The sum is formed in fp32 and tested against the rounding ties of bf16 with a rigorous bound of
 * its error; values within the bound of a tie are recomputed with exact products and a float64
 * sum, which is exact for factors whose products span less than 2^30 in magnitude.
 * Errors: NF4_ERR_NULL, NF4_ERR_SHAPE (also a weight with fp32 scales), NF4_ERR_ALIGN,
 * NF4_ERR_RANK, NF4_ERR_HIP. */
int qlora_merge(const nf4_weight *W, const uint16_t *A, const uint16_t *B, int32_t r, float scale,
                uint16_t *out, hipStream_t stream);

/* ---- Codebook and blocksize variants, and scales without double quantisation ("QLoRA, explained",
 * A toy run, with the codebooks above and blocksizes from 16 to 4096; Double quantisation, whose
 * baseline keeps one fp32 absmax per block). The same storage layout as above with another
 * codebook and blocksize: packed[j] holds the indices of elements 2j (high nibble) and 2j+1 (low
 * nibble); one fp32 absmax per block of `blocksize` consecutive values. Double quantisation of
 * those scales is nf4_double_quant on the absmax array (any length; groups of 256 blocks). At
 * blocksize 64 the result is an nf4_weight with that codebook. */

/* Writes the codebook's values, ascending, as fp32 (out[15] repeats the last code when there are
 * 15) and returns how many there are (15 or 16); a negative status for an unknown codebook. */
int q4_codebook_values(int32_t codebook, float out[16]);

/* Blockwise absmax quantisation to the exact nearest code (ties to the lower index; an all-zero
 * block takes the exact-zero code). numel a multiple of 64 and of blocksize; blocksize a power of
 * two in 16..4096. packed: numel/2 bytes; absmax: numel/blocksize floats. Inputs finite.
 * Errors: NF4_ERR_SHAPE (codebook, blocksize or numel), NF4_ERR_NULL, NF4_ERR_ALIGN. */
int q4_quantize(const float *w, int64_t numel, int32_t codebook, int32_t blocksize, uint8_t *packed,
                float *absmax, hipStream_t stream);

/* out[i] = bf16(fl32(q[idx_i] * s_b)), b the block of element i. Exactly one kind of scales:
 *   absmax != NULL, scale_q == scale_c2 == NULL: s_b = absmax[b] (fp32, no double quantisation);
 *   absmax == NULL: s_b = fl32(e4m3(scale_q[b]) * scale_c2[b / 256]) (double quantised).
 * Indices must be below the codebook's size. Errors: NF4_ERR_SHAPE, NF4_ERR_NULL (missing or
 * both kinds of scales), NF4_ERR_ALIGN. */
int q4_dequant(const uint8_t *packed, int64_t numel, int32_t codebook, int32_t blocksize, const float *absmax,
               const uint8_t *scale_q, const float *scale_c2, uint16_t *out, hipStream_t stream);

/* ---- The adapter update of a training step ("QLoRA, explained", The algorithm, step by step, and
 * Minimal implementation): the adapter gradients are clipped by their global L2 norm (0.3 in the
 * original runs), then AdamW with 32-bit state updates A and B only. AdamW as torch documents it
 * (decoupled weight decay); for clipped gradient g = c * grad at step t = 1, 2, ...:
 *   p <- p * (1 - lr*weight_decay);  m <- beta1*m + (1-beta1)*g;  v <- beta2*v + (1-beta2)*g^2;
 *   p <- p - (lr / (1 - beta1^t)) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps),
 * c = min(1, max_grad_norm / (norm + 1e-6)) (1 when max_grad_norm <= 0), norm the L2 norm over
 * every gradient value of every tensor of the plan. Paged and 8-bit optimiser state are not
 * provided. */
typedef struct {
  float lr;             /* learning rate (the pages use 2e-4); >= 0 */
  float beta1, beta2;   /* in [0, 1) */
  float eps;            /* > 0 */
  float weight_decay;   /* >= 0 */
  float max_grad_norm;  /* clipping threshold; <= 0 disables clipping */
} qlora_adamw_config;

/* Opaque: the device pointers and sizes of a set of adapter tensors, as a table of 4096-value
 * chunk descriptors in device memory, so that one step over any number of tensors is three
 * kernel launches. */
typedef struct qlora_adamw_plan qlora_adamw_plan;

/* Build a plan over `count` tensors (count >= 1). The arguments are HOST arrays of `count` entries:
 *   params      fp32 master weights (A and B of every adapted linear), updated in place
 *   grads       fp32 gradients of the same sizes
 *   exp_avg, exp_avg_sq   fp32 first and second moments, updated in place (zero before step 1)
 *   params_bf16 NULL, or bf16 buffers that receive the new weights rounded to nearest even (the A
 *               and B the next forward reads); entries may be NULL
 *   numel       values per tensor: > 0 and a multiple of 4
 * Every pointer 16-byte aligned (bf16 buffers: 8-byte). The tensors must stay allocated at these
 * addresses while the plan is used. Allocates device memory on the current device (about 12 bytes
 * per 1024 values) and blocks until the table is uploaded. *out receives the plan, or NULL.
 * Errors: NF4_ERR_NULL, NF4_ERR_SHAPE (count or numel), NF4_ERR_ALIGN, NF4_ERR_HIP (allocation). */
int qlora_adamw_plan_create(int64_t count, float *const *params, const float *const *grads,
                            float *const *exp_avg, float *const *exp_avg_sq, uint16_t *const *params_bf16,
                            const int64_t *numel, qlora_adamw_plan **out);

/* One clipped AdamW step over every tensor of the plan, on `stream`, on the plan's device:
 * the squared gradient norm (partial sums in double over 16384-value groups, added in a fixed
 * order, so it is reproducible bit for bit), then the elementwise update. grad_norm (device
 * double, may be NULL) receives the norm before clipping. step counts from 1. Steps on one plan
 * must not overlap (they share the plan's scratch).
 * Errors: NF4_ERR_NULL, NF4_ERR_SHAPE (step < 1 or a config value out of range), NF4_ERR_ALIGN,
 * NF4_ERR_HIP (launch failure, or a device other than the plan's is current). */
int qlora_adamw_plan_step(const qlora_adamw_plan *plan, const qlora_adamw_config *cfg, int64_t step,
                          double *grad_norm, hipStream_t stream);

/* Free the plan (its device memory). No step on it may still be running. NULL is a no-op. */
int qlora_adamw_plan_destroy(qlora_adamw_plan *plan);

/* Workspace bytes that qlora_linear_fwd and qlora_linear_bwd need for these sizes (the larger of
 * the two). Returns 0 for invalid sizes. */
size_t qlora_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r);

/* Bytes of an NF4 + double-quantised weight with numel values: numel/2 + numel/64 + 4*ceil(numel/16384).
 * Returns -1 if numel is negative or not a multiple of 64. */
int64_t nf4_storage_bytes(int64_t numel);

/* Host copy of the 16 float32 NF4 codes the kernels use (ascending, index 7 is 0). */
void nf4_codebook(float out[16]);

/* Static description of a status code. */
const char *nf4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
