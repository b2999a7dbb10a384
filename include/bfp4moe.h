/*
 * bfp4moe: NVFP4 routed mixture-of-experts expert computation on AMD MI355X (gfx950).
 *
 * C ABI.  Every pointer argument named as a device pointer refers to device memory owned by the
 * caller; the library keeps no reference after a call returns, allocates no device memory on the
 * paths below and never synchronizes the stream.  All work is enqueued asynchronously on
 * `stream` (a hipStream_t handle; NULL means the default stream).
 *
 * Every entry point returns a bfp4_status.  Arguments are validated on the host from sizes,
 * pointer values and alignment only (device memory is never read for validation), so an error
 * is reported before anything is enqueued.  Device-side preconditions (documented per call) are
 * not checked.
 *
 * Sources, cited by page title and section:
 *   [cuDNN]   FlashInfer, "flashinfer.fused_moe.CudnnGroupedGemmNvfp4Config" (bullet list)
 *   [MCore]   NVIDIA Megatron-Core, "core.inference.moe.flashinfer_nvfp4" (module text, data, API)
 *   [Alpha]   FlashInfer, "flashinfer.fused_moe.alphamoe_nvfp4_aligned_moe" (signature, layout
 *             paragraph, parameter list, notes)
 *   [vLLM]    vLLM, "vllm.model_executor.layers.quantization.utils.flashinfer_utils"
 *   [Frost]   FlashInfer, "flashinfer.fused_moe.FrostLowLatencyConfig" (numerics paragraphs)
 *
 * Formats shared by all calls:
 *   NVFP4 row of C values = packed E2M1 bytes [C/2] (two values per byte, even logical value in
 *   the low nibble [Alpha, layout]) + E4M3FN scale bytes [C/16], one per 16 consecutive values,
 *   linear (not swizzled) [Alpha, layout] + one FP32 *decode* scale per row or matrix
 *   [vLLM, quantize_nvfp4_per_token_input]; value = e2m1 * e4m3 * decode_scale.
 *   BF16 values are passed as uint16_t bit patterns.
 */
#ifndef BFP4MOE_H
#define BFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BFP4_OK = 0,
  BFP4_ERR_NULL = -1,        /* a required pointer is NULL */
  BFP4_ERR_SHAPE = -2,       /* a size is out of range or not a required multiple */
  BFP4_ERR_ALIGN = -3,       /* a pointer or row stride is not aligned as required */
  BFP4_ERR_BLOCK_M = -4,     /* block_m < 8 or not a multiple of 8 [Alpha, block_m] */
  BFP4_ERR_CAPACITY = -5,    /* plan capacity below bfp4_plan_capacity() */
  BFP4_ERR_WORKSPACE = -6,   /* workspace or panel buffer smaller than required */
  BFP4_ERR_OVERLAP = -7,     /* out overlaps an input [Alpha, out] */
  BFP4_ERR_EXPERTS = -8,     /* expert range invalid */
  BFP4_ERR_MODE = -9,        /* unknown activation or scale mode */
  BFP4_ERR_SCALAR = -10,     /* a scalar is not finite / not positive */
  BFP4_ERR_DEVICE = -11,     /* no HIP device, or the current device is not gfx950 */
  BFP4_ERR_LAUNCH = -12      /* a kernel launch failed */
} bfp4_status;

/* Typed activations [cuDNN, activation bullet: SwiGLU with default scalars, GeGLU, GELU, ReLU,
 * SiLU, Identity; Megatron-Core flashinfer_nvfp4: squared ReLU].  SWIGLU and GEGLU are gated:
 * W1 holds [gate; up] (N1 = 2*I) and h = act(gate) * up; the others use one projection (N1 = I).
 * silu(x) = x / (1 + e^-x); gelu(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), the erf form. */
typedef enum {
  BFP4_ACT_SWIGLU = 0,    /* silu(gate) * up */
  BFP4_ACT_RELU2 = 1,     /* max(x, 0)^2 */
  BFP4_ACT_GEGLU = 2,     /* gelu(gate) * up */
  BFP4_ACT_GELU = 3,      /* gelu(x) */
  BFP4_ACT_RELU = 4,      /* max(x, 0) */
  BFP4_ACT_SILU = 5,      /* silu(x) */
  BFP4_ACT_IDENTITY = 6   /* x */
} bfp4_act;
typedef enum {
  BFP4_SCALE_PER_ROW = 0,
  BFP4_SCALE_PER_GROUP = 1,
  BFP4_SCALE_FIXED = 2
} bfp4_scale_mode;
/* Routing weights [cuDNN, routing weights bullet: unpacked FP32 or BF16]: FP32 values, or BF16
 * bit patterns, which the combine uses as their exact FP32 values. */
typedef enum { BFP4_WEIGHTS_F32 = 0, BFP4_WEIGHTS_BF16 = 1 } bfp4_weights_dtype;
/* Expert weight formats of the weight-only mode [Frost, FP4 weight-only paragraph]: NVFP4 (E2M1
 * with linear E4M3 scales per 16 values and one FP32 scale per expert) or MXFP4 (E2M1 with
 * UE8M0 power-of-two scales per 32 values, 127 encoding 1.0 [vLLM align_moe_weights_for_fi]). */
typedef enum { BFP4_FORMAT_NVFP4 = 0, BFP4_FORMAT_MXFP4 = 1 } bfp4_weight_format;

/* Human-readable name of a status code (static storage). */
const char* bfp4_status_string(int status);

/* Library version string (static storage). */
const char* bfp4_version(void);

/* ----------------------------------------------------------------------------------------------
 * Routing plan [Alpha, plan paragraph and parameters sorted_token_ids / expert_ids /
 * num_tokens_post_padded; cuDNN, permutation and expert-parallelism bullets].
 *
 * Slot (t, j) of topk_ids [M, top_k] is routed here when its id lies in
 * [local_expert_offset, local_expert_offset + num_local_experts) (and in [0, num_experts));
 * other ids, including -1, are unrouted [cuDNN EP bullet; MCore "-1 contribute zero"; Frost].
 * The plan lists routed slots by local expert, ascending, each expert segment padded to a
 * multiple of block_m; inside a segment the flat slot indices f = t*top_k + j ascend.
 *   sorted_token_ids [capacity]: f for routed entries, M*top_k (sentinel) for padding and for
 *                                every entry at or past the extent;
 *   expert_ids [capacity / block_m]: local expert id of each block, -1 past the extent;
 *   num_tokens_post_padded [1]: the extent P (a multiple of block_m);
 *   token_to_row [M, top_k]: plan row of each slot, -1 when unrouted.
 * capacity must be >= bfp4_plan_capacity(M, top_k, num_local_experts, block_m), a multiple of
 * block_m; the extent never exceeds it.  Ids are int32, device pointers, contiguous.
 * workspace: device scratch of at least bfp4_plan_workspace_size() bytes (may be NULL when that
 * size is 0).  Device precondition: none (any id values are accepted; duplicates inside a token,
 * which the pages forbid [cuDNN, topk_ids bullet], still give a valid stable plan).
 * Limits: num_local_experts <= 1024, M*top_k < 2^31.
 * ---------------------------------------------------------------------------------------------- */
size_t bfp4_plan_capacity(int64_t M, int top_k, int num_local_experts, int block_m);
size_t bfp4_plan_workspace_size(int64_t M, int top_k, int num_local_experts);
int bfp4_moe_plan(const int32_t* topk_ids, int64_t M, int top_k, int num_experts,
                  int local_expert_offset, int num_local_experts, int block_m,
                  int32_t* sorted_token_ids, int32_t* expert_ids, int32_t* num_tokens_post_padded,
                  int32_t* token_to_row, size_t capacity, void* workspace, size_t workspace_bytes,
                  void* stream);

/* ----------------------------------------------------------------------------------------------
 * NVFP4 quantization of a BF16 matrix x [rows, cols] (row stride in elements)
 * [MCore: one FP32 scale per token / per expert matrix; cuDNN: intermediate with a global scale
 * of one; vLLM: the returned scale is the decode scale; Alpha: packing and linear scales].
 *   mode PER_ROW:   one scale per row (activations); dec_scale [rows].
 *   mode PER_GROUP: one scale per group of group_rows consecutive rows (one expert matrix);
 *                   dec_scale [rows / group_rows].
 *   mode FIXED:     encode scale fixed_encode_scale for every row; dec_scale may be NULL, else
 *                   receives [1] = 1/fixed_encode_scale.
 * Arithmetic (FP32, round to nearest even, no fused multiply-add):
 *   s_enc = 2688 / amax (1 when amax == 0, infinity clamped to FLT_MAX); dec = 1 / s_enc;
 *   per 16-block: sf = e4m3_rne_sat((bmax * s_enc) / 6); inv = sf ? s_enc / sf : 0;
 *   code = e2m1_rne_sat(x * inv), ties to the even code, sign bit copied from x.
 * Outputs (device, contiguous): q [rows, cols/2], sf [rows, cols/16].
 * Requirements: cols % 32 == 0; row_stride >= cols and % 8 == 0; x 16-byte aligned, q 8-byte
 * aligned, dec_scale 4-byte aligned; q and sf must not overlap x;
 * workspace >= bfp4_quantize_workspace_size(rows, mode, group_rows) (PER_GROUP keeps the group
 * maxima there).  Device preconditions: x finite; every row (group) maximum is 0 or >= 2^-106.
 * ---------------------------------------------------------------------------------------------- */
size_t bfp4_quantize_workspace_size(int64_t rows, int mode, int64_t group_rows);
int bfp4_quantize_nvfp4(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t row_stride,
                        int mode, int64_t group_rows, float fixed_encode_scale, uint8_t* q,
                        uint8_t* sf, float* dec_scale, void* workspace, size_t workspace_bytes,
                        void* stream);

/* ----------------------------------------------------------------------------------------------
 * Plan and activation quantization of one batch in one call [Alpha, plan paragraph; MCore,
 * quantize_routed_nvfp4_input; vLLM quantize_nvfp4_per_token_input].  Writes exactly what
 * bfp4_moe_plan(topk_ids, M, ...) followed by bfp4_quantize_nvfp4(x_bf16, M, H, row_stride,
 * BFP4_SCALE_PER_ROW, ...) write, with the same arguments, contracts and errors (plan_workspace
 * is the plan's workspace; x_bf16 [M rows, row_stride] BF16, q [M, H/2], sf [M, H/16],
 * dec_scale [M]).  The two are independent, so when the plan fits one workgroup
 * (M * top_k <= 2048 slots, the decode sizes) they run as one kernel launch, which saves a
 * launch on the latency-bound decode path; larger batches run the two calls' kernels in order.
 * ---------------------------------------------------------------------------------------------- */
int bfp4_moe_plan_quantize(const int32_t* topk_ids, int64_t M, int top_k, int num_experts,
                           int local_expert_offset, int num_local_experts, int block_m,
                           int32_t* sorted_token_ids, int32_t* expert_ids,
                           int32_t* num_tokens_post_padded, int32_t* token_to_row,
                           size_t capacity, void* plan_workspace, size_t plan_workspace_bytes,
                           const uint16_t* x_bf16, int64_t H, int64_t row_stride, uint8_t* q,
                           uint8_t* sf, float* dec_scale, void* stream);

/* ----------------------------------------------------------------------------------------------
 * Permutation of quantized token rows into plan order [cuDNN, permutation bullet]:
 * for plan row r < extent with entry f < M*top_k, row r of the outputs is token f / top_k
 * (q_perm [capacity, H/2], sf_perm [capacity, H/16], s_perm [capacity]); sentinel rows and rows
 * at or past the extent are zero.  Inputs: q [M, H/2], sf [M, H/16], dec_scale [M] (device).
 * Requirements: H % 32 == 0; all byte pointers 16-byte aligned.  Device precondition: plan
 * produced for this M and top_k.
 * ---------------------------------------------------------------------------------------------- */
int bfp4_moe_permute(const uint8_t* q, const uint8_t* sf, const float* dec_scale, int64_t M,
                     int64_t H, int top_k, const int32_t* sorted_token_ids,
                     const int32_t* num_tokens_post_padded, size_t capacity, uint8_t* q_perm,
                     uint8_t* sf_perm, float* s_perm, void* stream);

/* ----------------------------------------------------------------------------------------------
 * Expert weights [MCore prepare_routed_nvfp4_weights; Alpha gemm1/gemm2 weight layouts].
 * Input: linear NVFP4 weights of num_local_experts experts, as bfp4_quantize_nvfp4 writes them
 * with one scale per expert matrix:
 *   w1_q [E, N1, H/2], w1_sf [E, N1, H/16] with N1 = 2*I in [gate; up] row order (gated) or I;
 *   w2_q [E, H, I/2],  w2_sf [E, H, I/16].
 * Output: `panels`, an opaque device buffer of bfp4_panel_bytes() bytes holding the same values
 * rearranged for the gfx950 kernels (gate/up row groups interleaved, K-blocked 1 KiB tiles, scales
 * grouped per 512 K values).  Requirements: H % 256 == 0, I % 128 == 0, all pointers 16-byte
 * aligned.  Runs once at load; the raw weights are not needed afterwards.
 * ---------------------------------------------------------------------------------------------- */
size_t bfp4_panel_bytes(int num_local_experts, int64_t H, int64_t I, int gated);
int bfp4_prepare_weights(const uint8_t* w1_q, const uint8_t* w1_sf, const uint8_t* w2_q,
                         const uint8_t* w2_sf, int num_local_experts, int64_t H, int64_t I,
                         int gated, void* panels, size_t panels_bytes, void* stream);

/* ----------------------------------------------------------------------------------------------
 * The fused expert computation [Alpha: gate/up GEMM, SwiGLU, requantization, down GEMM on a
 * pre-aligned plan; cuDNN: pipeline, finalize / unfinalized triple; Frost: rounding points].
 *
 * Per valid plan row r (entry f < M*top_k, token t = f / top_k, local expert e of r's block):
 *   pre[n] = (sum_h x[t,h] * W1_e[n,h]) * a_dec[t] * alpha1_{gate|up}[e]   (FP32 accumulate;
 *            gate rows n < I use alpha1_gate, up rows alpha1_up; non-gated uses alpha1_up)
 *   h[i]   = bf16(act(pre[i]) * pre[I+i])  (gated: SwiGLU, GeGLU)  or  bf16(act(pre[i]))
 *            (ReLU^2, GELU, ReLU, SiLU, Identity); act is the bfp4_act code
 *   hq     = NVFP4 of h with fixed encode scale c2 (the quantizer's FIXED mode)
 *   y[k]   = bf16((sum_i hq[i] * W2_e[k,i]) * (1/c2) * alpha2[e])
 * Finalize (do_finalize != 0): for every token t,
 *   out[t,k] = bf16(f32(out[t,k]) + sum_{j ascending, token_to_row[t,j] >= 0}
 *              fl32(fl32(w[t,j] * y[row,k]) [* rsf]))   -- each product and sum rounded to FP32,
 *   no fused multiply-add; unrouted slots are skipped without reading their weights [Frost].
 *   out accumulates: zero it first for a fresh result [Alpha, out].
 * Unfinalized (do_finalize == 0): gemm2_out [capacity, H] receives y at every routed row (rows
 *   not named by token_to_row are left unwritten); with topk_weights and token_to_row this is the
 *   [gemm2_out, expert_weights, token_to_row] triple [cuDNN, finalize bullet]; out is untouched.
 *
 * Arguments (device pointers unless noted):
 *   a_q [M, H/2], a_sf [M, H/16], a_dec [M]: NVFP4 activations (bfp4_quantize_nvfp4 PER_ROW);
 *   panels: from bfp4_prepare_weights for (num_local_experts, H, I, gated), gated matching act
 *   (panels_bytes below the size for act gives BFP4_ERR_WORKSPACE);
 *   alpha1_gate, alpha1_up, alpha2 [num_local_experts] FP32;  c2 (host) > 0, finite;
 *   sorted_token_ids, expert_ids, num_tokens_post_padded, token_to_row: a plan from
 *   bfp4_moe_plan for the same M, top_k, num_local_experts and block_m, with this capacity;
 *   topk_weights [M, top_k] FP32 (weights_dtype BFP4_WEIGHTS_F32, 4-byte aligned) or BF16
 *   (BFP4_WEIGHTS_BF16, 2-byte aligned); another weights_dtype gives BFP4_ERR_MODE;
 *   routed_scaling_factor (host) finite;
 *   out [M, H] BF16 (16-byte aligned, must not overlap any input or the workspace) -- used
 *   when do_finalize;
 *   gemm2_out [capacity, H] BF16 (16-byte aligned, must not overlap any input or the
 *   workspace) -- required when !do_finalize, else may be NULL;
 *   debug (may be NULL): optional copies of internal values for verification.
 *   workspace: >= bfp4_workspace_size(M, H, I, top_k, num_local_experts, block_m, do_finalize).
 * Requirements: H % 256 == 0 and H >= 256 [Alpha, notes]; I % 128 == 0 [cuDNN, sizes bullet];
 *   block_m >= 8, % 8 == 0 [Alpha, block_m]; pointers 16-byte aligned.  With block_m > 32 (the
 *   tiled prefill kernels, which read exact FP16 copies of their token operands through 32-bit
 *   buffer offsets) also M*H*2 < 2^31 and capacity*I*2 < 2^31 bytes, and one expert's panel
 *   of each matrix (bfp4_panel_bytes(1, ...) splits into the two) below 2^31 bytes, else
 *   BFP4_ERR_SHAPE (split such a batch into several calls).  With block_m <= 32 (the decode
 *   kernels, which stage a plan block's routed rows whole in LDS) min(block_m, 32) rows of
 *   K/2 + K/16 bytes (rounded up to 16) plus 256 bytes must fit in 160 KiB for K = H and K = I
 *   (for H a multiple of 256: H <= 8960 at block_m 32, 18176 at 16, 36352 at 8), else
 *   BFP4_ERR_SHAPE.
 * Device preconditions: the plan's expert ids are < num_local_experts; token ids < M.
 * ---------------------------------------------------------------------------------------------- */
typedef struct {
  float* preact;        /* [capacity, N1] FP32 pre-activations (logical W1 row order) or NULL */
  uint16_t* inter;      /* [capacity, I] BF16 activation output or NULL */
  uint8_t* inter_q;     /* [capacity, I/2] requantized intermediate or NULL */
  uint8_t* inter_sf;    /* [capacity, I/16] its E4M3 scales or NULL */
  uint16_t* inter_f16;  /* block_m > 32 only: [capacity, I] FP16, 16-byte aligned, or NULL: the
                           exact FP16 decode of (inter_q, inter_sf) that the tiled down GEMM
                           reads as its token operand (the call uses this buffer in place of its
                           workspace copy); rows that are not routed are left unwritten; unused
                           (not written) when block_m <= 32 */
} bfp4_debug;

size_t bfp4_workspace_size(int64_t M, int64_t H, int64_t I, int top_k, int num_local_experts,
                           int block_m, int do_finalize);
int bfp4_fused_moe_nvfp4(const uint8_t* a_q, const uint8_t* a_sf, const float* a_dec,
                         const void* panels, size_t panels_bytes, const float* alpha1_gate,
                         const float* alpha1_up, const float* alpha2, float c2,
                         const int32_t* sorted_token_ids, const int32_t* expert_ids,
                         const int32_t* num_tokens_post_padded, const int32_t* token_to_row,
                         size_t capacity, const void* topk_weights, int weights_dtype,
                         int64_t M, int64_t H, int64_t I, int num_local_experts, int top_k,
                         int block_m, int act,
                         float routed_scaling_factor, int do_finalize, uint16_t* out,
                         uint16_t* gemm2_out, const bfp4_debug* debug, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------------------------------
 * The fused expert computation without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, contract and results as bfp4_fused_moe_nvfp4 (the same kernels
 * run), minus workspace / workspace_bytes: the workspace lives in a static device array of
 * BFP4_NOALLOC_SCRATCH_BYTES (64 MiB) that every GPU the library runs on holds until the
 * process ends.  A call whose bfp4_workspace_size(...) exceeds it returns BFP4_ERR_WORKSPACE
 * before touching the device (e.g. the decode shapes M=8, H=7168, I=2048, 256 experts fit; a
 * 4096-token prefill does not: use the workspace entry point).  The call allocates nothing and
 * calls no allocating routine.  Every call on one GPU uses that GPU's one array, so calls that
 * overlap in time on one GPU (other streams or threads) race and give undefined results: order
 * them.  The array keeps the last call's contents; nothing in it needs to start at zero (the
 * kernels clear their counters themselves).  The first call on each device looks the array's
 * address up (hipGetSymbolAddress, with that device current); make it outside a stream capture.
 * ---------------------------------------------------------------------------------------------- */
#define BFP4_NOALLOC_SCRATCH_BYTES (64u << 20)
int bfp4_fused_moe_nvfp4_noalloc(const uint8_t* a_q, const uint8_t* a_sf, const float* a_dec,
                                 const void* panels, size_t panels_bytes,
                                 const float* alpha1_gate, const float* alpha1_up,
                                 const float* alpha2, float c2, const int32_t* sorted_token_ids,
                                 const int32_t* expert_ids,
                                 const int32_t* num_tokens_post_padded,
                                 const int32_t* token_to_row, size_t capacity,
                                 const void* topk_weights, int weights_dtype, int64_t M,
                                 int64_t H, int64_t I, int num_local_experts, int top_k,
                                 int block_m, int act, float routed_scaling_factor,
                                 int do_finalize, uint16_t* out, uint16_t* gemm2_out,
                                 const bfp4_debug* debug, void* stream);

/* ----------------------------------------------------------------------------------------------
 * MXFP4 quantization of BF16 rows [Frost, FP4 weight-only paragraph: E8M0 K32 scales;
 * prepare_mxfp4_weight_only_weights: linear E8M0 scales per 32 K values; vLLM
 * align_moe_weights_for_fi: UE8M0 block scales, 127 = 1.0].  The recipe is not on the pages;
 * reading taken (the OCP microscaling one): per 32 consecutive values of a row, with amax their
 * largest magnitude, the shared exponent X = floor(log2(amax)) - 2 (clamped to [-127, 127]; amax
 * 0 or below the FP32 normal range gives code 0) is stored as the UE8M0 code X + 127, and each
 * value as the E2M1 code nearest to x * 2^-X (ties to the even code, saturating at 6, sign bit
 * copied).  Packing as NVFP4: two codes per byte, even value in the low nibble.
 *   x_bf16 [rows, row_stride >= cols] (16-byte aligned, row_stride % 8 == 0), cols % 32 == 0;
 *   q [rows, cols/2] (16-byte aligned), sf [rows, cols/32]; q and sf must not overlap x.
 * ---------------------------------------------------------------------------------------------- */
int bfp4_quantize_mxfp4(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t row_stride,
                        uint8_t* q, uint8_t* sf, void* stream);

/* Panels from linear MXFP4 weights (bfp4_quantize_mxfp4 of each expert matrix's rows): W1
 * [E, N1, H/2] + [E, N1, H/32], W2 [E, H, I/2] + [E, H, I/32]; the same panel layout and size as
 * bfp4_prepare_weights (each UE8M0 code fills the two 16-value scale slots).  For
 * bfp4_fused_moe_w4a16 with BFP4_FORMAT_MXFP4 (alphas of 1) and for bfp4_fused_moe_mx. */
int bfp4_prepare_weights_mxfp4(const uint8_t* w1_q, const uint8_t* w1_sf, const uint8_t* w2_q,
                               const uint8_t* w2_sf, int num_local_experts, int64_t H, int64_t I,
                               int gated, void* panels, size_t panels_bytes, void* stream);

/* ----------------------------------------------------------------------------------------------
 * MXFP8 quantization of BF16 rows (the activation format of the MX mode below) [Frost, MX
 * paragraph: MXFP4 or MXFP8 weights with MXFP8 inputs].  Reading taken (the OCP microscaling
 * recipe, as for MXFP4 with E4M3's largest exponent 8 in place of E2M1's 2): per 32 consecutive
 * values with amax their largest magnitude, the UE8M0 code X + 127 of X = floor(log2(amax)) - 8
 * (clamped to [-127, 127]; amax 0 or below the FP32 normal range gives code 0), and each value
 * as the E4M3FN code nearest to x * 2^-X (ties to the even code, saturating at 448, sign bit
 * copied).
 *   x_bf16 [rows, row_stride >= cols] (16-byte aligned, row_stride % 8 == 0), cols % 32 == 0;
 *   q [rows, cols] E4M3 bytes (16-byte aligned), sf [rows, cols/32]; neither may overlap x.
 * ---------------------------------------------------------------------------------------------- */
int bfp4_quantize_mxfp8(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t row_stride,
                        uint8_t* q, uint8_t* sf, void* stream);

/* ----------------------------------------------------------------------------------------------
 * The fused expert computation with MXFP4 weights on MXFP8 activations [Frost, MX paragraph:
 * the same typed activations, activation output and expert outputs rounded to BF16, ordered FP32
 * combine, an intermediate quantization contract of the MX mode's own].  On gfx950's block-scaled
 * MFMA (FP4 weights x FP8 activations, E8M0 scales per 32 values), no decode of either operand.
 * Readings taken: MX weights and activations carry no FP32 global scales; the BF16 intermediate
 * is quantized to MXFP8 (bfp4_quantize_mxfp8's recipe, per 32 values of a row) before GEMM2.
 * Per valid plan row r (token t, local expert e):
 *   pre[n] = sum_h a[t,h] * W1_e[n,h]          (exact products, FP32 accumulation; the
 *            instruction sums each 64-product chunk with an error of up to about 2^-13 of the
 *            chunk's sum of magnitudes, measured)
 *   h[i]   = bf16(act(pre[i]) * pre[I+i]) (gated) or bf16(act(pre[i]));  hq = MXFP8(h)
 *   y[k]   = bf16(sum_i hq[i] * W2_e[k,i]);   finalize / unfinalized as bfp4_fused_moe_nvfp4.
 * Arguments as bfp4_fused_moe_nvfp4, except: a_q [M, H] E4M3 bytes and a_sf [M, H/32] E8M0 from
 * bfp4_quantize_mxfp8 (no per-token scale); panels from bfp4_prepare_weights_mxfp4; no alphas
 * or c2; block_m <= 32 runs the decode kernels, block_m > 32 the tiled prefill kernels (which
 * need M*H and capacity*I below 2^31 bytes and one expert's panel of each matrix below 2^31
 * bytes, else BFP4_ERR_SHAPE); workspace >= bfp4_workspace_size_mx(...) bytes, 256-byte
 * aligned.  debug->preact [capacity, N1] FP32, debug->inter [capacity, I] BF16,
 * debug->inter_q [capacity, I] (the MXFP8 intermediate, 16-byte aligned) and debug->inter_sf
 * [capacity, I/32]; inter_f16 unused.
 * ---------------------------------------------------------------------------------------------- */
size_t bfp4_workspace_size_mx(int64_t M, int64_t H, int64_t I, int top_k, int num_local_experts,
                              int block_m, int do_finalize);
int bfp4_fused_moe_mx(const uint8_t* a_q, const uint8_t* a_sf, const void* panels,
                      size_t panels_bytes, const int32_t* sorted_token_ids,
                      const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                      const int32_t* token_to_row, size_t capacity, const void* topk_weights,
                      int weights_dtype, int64_t M, int64_t H, int64_t I, int num_local_experts,
                      int top_k, int block_m, int act, float routed_scaling_factor,
                      int do_finalize, uint16_t* out, uint16_t* gemm2_out,
                      const bfp4_debug* debug, void* workspace, size_t workspace_bytes,
                      void* stream);

/* ----------------------------------------------------------------------------------------------
 * FP4 weight-only forward on BF16 activations, NVFP4 or MXFP4 weights [Frost, FP4 weight-only
 * paragraph: canonical E2M1 weights with linear E4M3 K16 scales and one FP32 scale per expert
 * (NVFP4) or E8M0 K32 scales (MXFP4); BF16 input,
 * pre-activation and intermediate rounding; BF16 expert outputs; the same combine].  Decode-sized
 * plans only (block_m <= 32, else BFP4_ERR_BLOCK_M).
 * Per valid plan row r (entry f < M*top_k, token t = f / top_k, local expert e of r's block):
 *   pre[n] = (sum_h x[t,h] * W1_e[n,h]) * alpha1_{gate|up}[e]     (FP32 accumulate of exact
 *            products: BF16 x E2M1 x E4M3), then p[n] = bf16(pre[n]);
 *   h[i]   = bf16(act(p[i]) * p[I+i])  (gated)  or  bf16(act(p[i]))  (one projection);
 *   y[k]   = bf16((sum_i h[i] * W2_e[k,i]) * alpha2[e]);
 * then the combine (or the unfinalized triple) exactly as bfp4_fused_moe_nvfp4.
 * Arguments as bfp4_fused_moe_nvfp4, except: x_bf16 [M rows, row_stride >= H elements,
 * row_stride % 8 == 0] BF16 activations in place of a_q/a_sf/a_dec, no c2; weight_format
 * (bfp4_weight_format) names how the panels were prepared (bfp4_prepare_weights or
 * bfp4_prepare_weights_mxfp4; MXFP4 is exact for scale codes 2..252, where every product stays
 * in BF16's normal range; another value gives BFP4_ERR_MODE); debug->preact gets
 * pre (FP32, before the BF16 rounding), debug->inter h (BF16); inter_q, inter_sf and inter_f16
 * are unused.
 * workspace: >= bfp4_workspace_size_w4a16(...) bytes, 256-byte aligned.
 * ---------------------------------------------------------------------------------------------- */
size_t bfp4_workspace_size_w4a16(int64_t M, int64_t H, int64_t I, int top_k,
                                 int num_local_experts, int block_m, int do_finalize);
int bfp4_fused_moe_w4a16(const uint16_t* x_bf16, int64_t row_stride, const void* panels,
                         size_t panels_bytes, int weight_format, const float* alpha1_gate,
                         const float* alpha1_up,
                         const float* alpha2, const int32_t* sorted_token_ids,
                         const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                         const int32_t* token_to_row, size_t capacity, const void* topk_weights,
                         int weights_dtype, int64_t M, int64_t H, int64_t I,
                         int num_local_experts, int top_k, int block_m, int act,
                         float routed_scaling_factor, int do_finalize, uint16_t* out,
                         uint16_t* gemm2_out, const bfp4_debug* debug, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------------------------------
 * Finalize an unfinalized triple [cuDNN finalize bullet; Frost combine contract]: the combine of
 * bfp4_fused_moe_nvfp4 applied to gemm2_out [rows, H], topk_weights [M, top_k] (FP32 or BF16 by
 * weights_dtype, as in bfp4_fused_moe_nvfp4) and token_to_row [M, top_k], accumulating into
 * out [M, H].  Bit-identical to the finalized path.
 * Requirements: H % 8 == 0; gemm2_out and out 16-byte aligned, token_to_row 4-byte, the weights
 * aligned to their element size; out must not overlap topk_weights or token_to_row (checked)
 * nor the gemm2_out rows token_to_row names (not checked: their number is not an argument).
 * ---------------------------------------------------------------------------------------------- */
int bfp4_moe_finalize(const uint16_t* gemm2_out, const void* topk_weights, int weights_dtype,
                      const int32_t* token_to_row, int64_t M, int64_t H, int top_k,
                      float routed_scaling_factor, uint16_t* out, void* stream);

/* ----------------------------------------------------------------------------------------------
 * Unpack packed routing [cuDNN, routing weights bullet: packed, or unpacked FP32 / BF16; Frost,
 * numerics paragraph: packed routing scores keep their BF16 rounding].  The pages give no bit
 * layout; a packed slot here is one 32-bit word holding the score's BF16 bits in its high 16 bits
 * and the expert id as a two's-complement 16-bit integer in its low 16 bits (an empty slot, id
 * -1, has low half 0xFFFF).
 *   packed       [M, top_k] int32 (device, 4-byte aligned);
 *   topk_ids     [M, top_k] int32 out: the ids, sign-extended (device, 4-byte aligned);
 *   topk_weights [M, top_k] BF16 bit patterns out: the score bits unchanged (device, 2-byte
 *                aligned).
 * The outputs are the routing inputs of bfp4_moe_plan / bfp4_moe_plan_quantize and, with
 * BFP4_WEIGHTS_BF16, of the fused calls and bfp4_moe_finalize; ids outside the routed range are
 * unrouted slots there whatever their score (NaN included).  The three arrays must not overlap
 * (checked).  Errors: BFP4_ERR_SHAPE (M < 0, top_k <= 0, M * top_k >= 2^31), BFP4_ERR_NULL,
 * BFP4_ERR_ALIGN, BFP4_ERR_OVERLAP, BFP4_ERR_DEVICE.  M == 0 returns BFP4_OK and launches nothing.
 * ---------------------------------------------------------------------------------------------- */
int bfp4_unpack_routing(const int32_t* packed, int64_t M, int top_k, int32_t* topk_ids,
                        uint16_t* topk_weights, void* stream);

/* ----------------------------------------------------------------------------------------------
 * Diagnostic outside the MoE path (no page defines it): the XOR of all 32-bit words of a device
 * buffer, read as a plain stream, which the benchmark times as the HBM read rate the GPU reaches
 * without any MoE work.  buf [bytes] (device, 16-byte aligned, bytes a multiple of 16);
 * partial [BFP4_XOR_PARTIALS] uint32 out (device, 4-byte aligned, not overlapping buf): one
 * word per reading wave, whose XOR is the buffer's.  Errors: BFP4_ERR_SHAPE, BFP4_ERR_NULL,
 * BFP4_ERR_ALIGN, BFP4_ERR_OVERLAP, BFP4_ERR_DEVICE.
 * ---------------------------------------------------------------------------------------------- */
#define BFP4_XOR_PARTIALS 16384
int bfp4_xor_checksum(const void* buf, size_t bytes, uint32_t* partial, void* stream);

/* ----------------------------------------------------------------------------------------------
 * Debug validation of device-side preconditions (off the hot path; the other calls never read
 * device memory to validate).  Each call overwrites report[3] (device, int32, 4-byte aligned, not
 * overlapping the inputs) on `stream`; read it back after the stream has reached it.
 *
 * bfp4_check_topk_ids [cuDNN, topk_ids bullet: each token's top_k experts are distinct; -1 marks
 * an empty slot]: topk_ids [M, top_k] int32.
 *   report[0] = tokens that hold some id >= 0 more than once;
 *   report[1] = ids outside [-1, num_experts);
 *   report[2] = smallest token index counted in either, or 2147483647 when there is none.
 * Duplicates still give a valid plan (bfp4_moe_plan ranks them stably); out-of-range ids are
 * unrouted.  Limits as bfp4_moe_plan.
 *
 * bfp4_check_plan [Alpha, plan paragraph and parameters]: the preconditions the fused calls place
 * on a plan they did not build, for this M, top_k, num_local_experts, block_m and capacity.
 *   report[0] = entries below the extent outside [0, M*top_k] (M*top_k is the padding sentinel);
 *   report[1] = blocks below the extent whose expert id is outside [0, num_local_experts);
 *   report[2] = 1 when the extent num_tokens_post_padded[0] is negative, above capacity or not a
 *               multiple of block_m (entries and blocks are then checked below the extent clamped
 *               to [0, capacity] and rounded down to a multiple of block_m), else 0.
 * A plan from bfp4_moe_plan reports {0, 0, 0}.
 * ---------------------------------------------------------------------------------------------- */
int bfp4_check_topk_ids(const int32_t* topk_ids, int64_t M, int top_k, int num_experts,
                        int32_t* report, void* stream);
int bfp4_check_plan(const int32_t* sorted_token_ids, const int32_t* expert_ids,
                    const int32_t* num_tokens_post_padded, size_t capacity, int64_t M, int top_k,
                    int num_local_experts, int block_m, int32_t* report, void* stream);

/* ----------------------------------------------------------------------------------------------
 * Kernel timing with HIP events (measurement support, off by default).
 * bfp4_profile_begin(capacity, name_prefix) creates `capacity` event pairs and starts recording
 * one pair around every kernel the library launches whose name starts with name_prefix (host
 * string; NULL or "" for every kernel): plan_*, quantize_* (quantize_rows, quantize_rows_group,
 * quantize_rows_fixed, quantize_mxfp4, with fill_u32 and group_amax), permute, prepare_weights,
 * tile_list, decode_tokens, gemm1_<activation>_{decode,prefill} (activation swiglu, relu2, geglu,
 * gelu, relu, silu or identity), gemm2_down_{decode,prefill}, the weight-only
 * gemm1_<activation>_w16_decode and gemm2_down_w16_decode, finalize, and the validators'
 * check_init, check_topk and check_plan.  The timer is process-wide state:
 * record from one host thread at a time, and not while a stream is being captured.
 * bfp4_profile_end() stops recording, waits for the
 * recorded events and writes one line per kernel name, "name count total_ms", into buf
 * (NUL-terminated, truncated to len).  Returns the number of kernels launched while recording,
 * or a negative status.
 * ---------------------------------------------------------------------------------------------- */
int bfp4_profile_begin(int capacity, const char* name_prefix);
int bfp4_profile_end(char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* BFP4MOE_H */
