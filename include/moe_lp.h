/*
 * moe_lp.h -- C ABI of the MI355X (gfx950) low-precision MoE expert forward.
 *
 * The operation (Orbit announcement, section 技术细节, "Active-expert-chunked
 * dequantization"): each token activates only the experts its router
 * selects; the selected experts are processed in fixed-size chunks whose
 * frozen low-precision weights are dequantized temporarily for a grouped
 * GEMM and released afterwards.  Weight formats: INT4 (Kimi INT4 base, same
 * page), FP8 E4M3 with [128,128] fp32 block scales and [1,128] activation
 * scales (NeMo RL FP8 post, Table 1), MXFP4 and NVFP4 (named as serving
 * formats in the mixed-precision sampler post, which defines neither; both
 * follow their public definitions).  The optional BF16 adapter is an OFT
 * orthogonal rotation of the expert input (Orbit analysis page, section on
 * why OFT matters); passing no adapter gives the frozen base, i.e. the
 * reference policy of that page.
 *
 * Conventions for every entry point
 *  - All array arguments are DEVICE pointers owned by the caller (e.g. torch
 *    tensors).  Only the descriptor structs live in host memory.  The library
 *    allocates nothing and keeps no state between calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued on it; no call synchronises the host and no call copies
 *    device data to the host.  Buffers must stay alive until the work is done.
 *  - Arguments are validated on the host before anything is enqueued; on any
 *    error the call returns a non-zero moe_status and enqueues nothing.  Kernel
 *    launch failures return MOE_ERR_DEVICE.  Non-finite logits or activations
 *    are a precondition violation (not checked).
 *  - Device pointers must be 16-byte aligned.
 *  - Row-major everywhere; weights are stored K-contiguous (Y = X W^T).
 */
#ifndef MOE_LP_H
#define MOE_LP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_LP_ABI_VERSION 6

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,    /* null pointer, bad shape, misalignment */
  MOE_ERR_UNSUPPORTED = 2,         /* valid but outside the supported limits */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3, /* ws_bytes < the matching *_workspace_bytes() */
  MOE_ERR_DEVICE = 4               /* a HIP launch reported an error */
} moe_status;

typedef enum {
  /* Two's-complement 4-bit codes, element 2i in the low nibble of byte i;
   * bf16 scale per (output row n, 32 consecutive k).  w = q * s.
   * Activations into the GEMMs: 16-bit floats (no activation quantization).
   * The GEMMs run on fp16 operands: w = q*s is exact in fp16 for bf16 scales
   * in [2^-17, 8188]; x (or x R_e with an adapter) and h = silu(gate)*up are
   * converted to fp16, exact in magnitude range [2^-14, 65504) for bf16 x.
   * Preconditions (not checked on the device): scales in that range and
   * |x|, |x R_e|, |h| < 65504 (larger values become infinite). */
  MOE_W_INT4_G32_BF16 = 1,
  /* OCP E4M3FN codes, one byte each; fp32 scale per [128,128] block
   * [n/128][k/128].  Activations (x and the SwiGLU output) are quantized to
   * E4M3 with an fp32 scale per [1,128] block: s = amax/448, q = RNE(v/s). */
  MOE_W_FP8_E4M3_B128 = 2,
  /* OCP MXFP4: E2M1 codes (low nibble first) with an E8M0 scale byte per
   * (n, 32 consecutive k).  Activations are quantized to MXFP8: E4M3 codes
   * with an E8M0 scale per 32, shared exponent floor(log2 amax) - 8. */
  MOE_W_MXFP4 = 3,
  /* As MOE_W_FP8_E4M3_B128 with power-of-two scales (the FP8 recipe's
   * power-of-two scaling-factor switches, NeMo RL FP8 post): weight block
   * scales must be exact powers of two (fp32, only their exponent is used);
   * activation scales are the smallest power of two >= fl32(amax/448).  The
   * GEMMs then apply both scales inside the block-scaled MFMA. */
  MOE_W_FP8_E4M3_B128_POW2 = 4,
  /* NVFP4 (named as a serving format in the mixed-precision sampler post;
   * this is the format's public definition): E2M1 codes (low nibble
   * first), an E4M3 scale byte per (n, 16 consecutive k), and one fp32
   * second-level scale per expert matrix (moe_scales.g13 / g2):
   * w = e2m1(q) * e4m3(s) * g.  Activations into the GEMMs: 16-bit floats,
   * as for INT4 (same range preconditions on x, x R_e and h; e2m1 * e4m3 is
   * exact in fp16 for every code, g multiplies the fp32 accumulators).
   * Forward, materialized forward and frozen-base backward. */
  MOE_W_NVFP4 = 5
} moe_wformat;

/* Storage order of the packed codes in w13 and w2 (every format). */
typedef enum {
  MOE_WL_ROWS = 0,   /* [E][N][K]: each output row's K codes contiguous */
  /* [E][N/16][K/128][16][B]: tiles of 16 rows x 128 codes, a row's 128
   * codes (B = 64 bytes of 4-bit codes in the usual nibble order, 128 bytes
   * of E4M3) contiguous within its tile, tiles K-fastest.  A GEMM step then
   * streams 1-2 KB runs instead of 64- or 128-byte pieces of rows K/2 or K
   * bytes apart.  Fused forward, materialized forward (its BF16 copy is in
   * rows either way) and frozen-base backward (the backward's transposed
   * copy is made from either order).  Written by moe_pack_weights_kblocked.
   * Scales keep their layout. */
  MOE_WL_KBLOCKED = 1
} moe_wlayout;

/* Layer description (host memory). */
typedef struct {
  /* T >= 0 (T = 0 is a no-op).  T*k*max(H, I)*2 must stay below 2^32 (the
   * grouped GEMMs address gathered activation rows with 32-bit byte offsets;
   * e.g. T <= 37449 at k = 8, H = 7168); larger: MOE_ERR_UNSUPPORTED. */
  int32_t num_tokens;
  int32_t hidden;      /* H: multiple of 256                                */
  int32_t inter;       /* I: multiple of 128 (expert intermediate size)     */
  int32_t num_experts; /* E: 1..1024                                        */
  int32_t top_k;       /* k: 1..min(16, E)                                  */
  int32_t wformat;     /* a moe_wformat value                               */
  int32_t oft_block;   /* 0: no adapter; 32: block-diagonal 32x32 rotation (every weight format) */
  int32_t tile_rows;   /* rows per grouped-GEMM tile: 0 = automatic, else 16, 32, 48, 64, 96, 128, 160 or 192 */
  int64_t adapter_expert_stride; /* elements between experts' R; 0 = one R shared by all */
  int32_t weight_layout;         /* a moe_wlayout value; other values: MOE_ERR_INVALID_ARGUMENT */
} moe_layer;

/* Packed expert weights.
 *   w13: [E][2I][H]  gate rows 0..I-1 then up rows I..2I-1 (packed bytes per format)
 *   w2 : [E][H][I]   down projection */
typedef struct {
  const void* w13;
  const void* w2;
} moe_qweights;

/* Scales, layouts per format.  Group scales (one per output row n and 32
 * or 16 consecutive k) are stored group-major, [K/32][N] per expert, so that
 * the scales of one K step for a block of output rows are contiguous:
 *   INT4 : s13 bf16 [E][H/32][2I],   s2 bf16 [E][I/32][H]
 *   FP8, FP8_POW2: s13 fp32 [E][2I/128][H/128], s2 fp32 [E][H/128][I/128]
 *   MXFP4: s13 u8   [E][H/32][2I],   s2 u8   [E][I/32][H]  (E8M0)
 *   NVFP4: s13 u8   [E][H/16][2I],   s2 u8   [E][I/16][H]  (E4M3, positive),
 *          g13, g2 fp32 [E] (device; 4-byte aligned).  g13 / g2 are read
 *          only for NVFP4 and may be NULL otherwise. */
typedef struct {
  const void* s13;
  const void* s2;
  const float* g13;
  const float* g2;
} moe_scales;

/* Routing result (all device arrays, caller-owned).  R = T*k.
 *   topk_ids[T][k]      int32, slots in descending logit order (ties: smaller id)
 *   topk_w[T][k]        fp32, softmax over the k selected logits
 *   expert_offsets[E+1] int32, exclusive scan of per-expert counts; [E] = R
 *   sorted_rows[R]      int32, permuted row -> flat pair t*k+j, stable in (t, j)
 *   row_of[R]           int32, flat pair -> permuted row (inverse of sorted_rows)
 *   active_experts[E]   int32, experts with >= 1 row in ascending id (first num_active valid)
 *   num_active[1]       int32 */
typedef struct {
  int32_t* topk_ids;
  float* topk_w;
  int32_t* expert_offsets;
  int32_t* sorted_rows;
  int32_t* row_of;
  int32_t* active_experts;
  int32_t* num_active;
} moe_route_out;

/* Workspace bytes moe_expert_forward needs for this layer (independent of
 * chunk_experts, which is accepted for symmetry; any value >= 1 gives the
 * same size).  Returns 0 for an invalid descriptor. */
size_t moe_workspace_bytes(const moe_layer* layer, int32_t chunk_experts);

/* Re-lays the codes from MOE_WL_ROWS (qweights, as described by
 * layer's dimensions and format; layer->weight_layout must be a valid value
 * but does not change what is read or written) into
 * MOE_WL_KBLOCKED: w13_out and w2_out (device, caller-owned, 16-byte
 * aligned, the same sizes as w13 and w2).  Bit-identical codes; a forward
 * with weight_layout = MOE_WL_KBLOCKED on the copy gives bit-identical
 * outputs.  Stream-ordered. */
moe_status moe_pack_weights_kblocked(const moe_layer* layer, const moe_qweights* qweights, void* w13_out,
                                     void* w2_out, void* stream);

/* Workspace bytes moe_route_permute needs (scan scratch only). */
size_t moe_route_workspace_bytes(const moe_layer* layer);

/* Rows per grouped-GEMM tile that moe_expert_forward uses for this layer
 * (layer->tile_rows if set, else the automatic choice); 0 if invalid. */
int32_t moe_tile_rows(const moe_layer* layer);

/* Router top-k + softmax over the selected logits, then the expert histogram,
 * exclusive scan and stable permutation by expert (Orbit announcement,
 * 技术细节: router-selected experts grouped dynamically).
 * logits: [T][E] fp32.  Outputs are bit-exact functions of the logits except
 * topk_w (fp32 softmax). */
moe_status moe_route_permute(const moe_layer* layer, const float* logits, const moe_route_out* out,
                             void* ws, size_t ws_bytes, void* stream);

/* The MoE expert forward (Orbit announcement, 技术细节, active-expert-chunked
 * dequantization): route, permute, then for each chunk of `chunk_experts`
 * consecutive active experts (ascending id) run the grouped
 * dequantize + GEMM1 (gate/up) + SwiGLU and the grouped dequantize + GEMM2
 * (down), and finally the weighted combine
 *   out[t] = sum_j topk_w[t][j] * y[t][j]   (fp32 sum in ascending j, bf16 out).
 * x: [T][H] bf16; logits: [T][E] fp32; adapter: NULL or bf16
 * R[E or 1][H/32][32][32] (x' = x R_e, rows of R index the input dim,
 * rotated per permuted row in fp32 and then given to the weight format's
 * GEMM1 input quantizer, as x is without an adapter); out: [T][H] bf16.  The launch count is fixed by (E, chunk_experts); the
 * result does not depend on chunk_experts.  ws: >= moe_workspace_bytes(). */
moe_status moe_expert_forward(const moe_layer* layer, const void* x_bf16, const float* logits,
                              const moe_qweights* qweights, const moe_scales* scales,
                              const void* adapter_bf16, int32_t chunk_experts, void* out_bf16,
                              void* ws, size_t ws_bytes, void* stream);

/* Stages reported by moe_expert_forward_timed. */
enum {
  MOE_STAGE_ROUTE = 0,   /* router top-k + softmax                          */
  MOE_STAGE_PERMUTE = 1, /* histogram, scan, stable scatter, tile lists      */
  MOE_STAGE_ACT = 2,     /* GEMM1 input: activation format and OFT rotation  */
  MOE_STAGE_GEMM1 = 3,   /* dequant + gate/up GEMM + SwiGLU                  */
  MOE_STAGE_GEMM2 = 4,   /* dequant + down GEMM (launch pairing: see below)  */
  MOE_STAGE_COMBINE = 5, /* weighted combine                                 */
  MOE_STAGE_DEQUANT = 6, /* materialized scheme only: chunk -> BF16 copy     */
  MOE_NUM_STAGES = 7
};

/* moe_expert_forward with per-stage timing, for measurement: a HIP event is
 * recorded on `stream` around every launch group, and the call synchronises
 * the stream before it returns (unlike moe_expert_forward).  stage_ms and
 * stage_launches are HOST arrays of MOE_NUM_STAGES entries, filled with the
 * summed event durations (milliseconds) and the number of launch groups of
 * each stage.  Same arguments, result and errors as moe_expert_forward.
 * The grouped GEMMs run one launch per chunk c = 0..n that does chunk c's GEMM1
 * together with chunk c-1's GEMM2 (n = number of chunks): launches 0..n-1
 * are reported under MOE_STAGE_GEMM1 and the last, GEMM2-only launch under
 * MOE_STAGE_GEMM2. */
moe_status moe_expert_forward_timed(const moe_layer* layer, const void* x_bf16, const float* logits,
                                    const moe_qweights* qweights, const moe_scales* scales,
                                    const void* adapter_bf16, int32_t chunk_experts, void* out_bf16,
                                    void* ws, size_t ws_bytes, void* stream, float* stage_ms,
                                    int32_t* stage_launches);

/* Workspace bytes moe_expert_forward_materialized needs: the routing arrays,
 * bf16 h [R][I] and y [R][H], the rotated input [R][H] bf16 when an adapter is
 * used, and one chunk's BF16 weight copy, min(chunk_experts, E) * 3*H*I * 2
 * bytes.  Returns 0 for an invalid descriptor or chunk_experts < 1. */
size_t moe_materialized_workspace_bytes(const moe_layer* layer, int32_t chunk_experts);

/* The materialized-chunk scheme (Orbit announcement, 技术细节: the chunk's
 * experts are dequantized temporarily to high precision, a grouped GEMM runs,
 * and the high-precision weights are released), for comparison with
 * moe_expert_forward.  Routing, permutation and combine are the same; then for
 * each chunk of chunk_experts consecutive active experts:
 *   1. dequantize the chunk's W13 and W2 into a BF16 copy in ws (each weight
 *      rounded once to bf16, nearest even),
 *   2. GEMM1 on bf16 MFMA: g, u = x~ W^T in fp32, h = silu(g) * u rounded to bf16,
 *   3. GEMM2: y = h W2^T in fp32, rounded to bf16,
 * and the next chunk overwrites the copy.  x~ is the bf16 token row, or x R_e
 * rounded to bf16 with the adapter; no activation quantizer is applied (the
 * copy is BF16, so the GEMMs are BF16 GEMMs for every weight format).
 * The copy's size, and so ws, grows with chunk_experts.
 * Same arguments and errors as moe_expert_forward, with
 * ws >= moe_materialized_workspace_bytes(layer, chunk_experts).  stage_ms and
 * stage_launches: both NULL (asynchronous, no host synchronisation), or both
 * HOST arrays of MOE_NUM_STAGES entries filled as by moe_expert_forward_timed
 * (the call then synchronises the stream); dequant launches are reported under
 * MOE_STAGE_DEQUANT, each chunk's GEMM1 and GEMM2 launch under GEMM1 and GEMM2. */
moe_status moe_expert_forward_materialized(const moe_layer* layer, const void* x_bf16, const float* logits,
                                           const moe_qweights* qweights, const moe_scales* scales,
                                           const void* adapter_bf16, int32_t chunk_experts, void* out_bf16,
                                           void* ws, size_t ws_bytes, void* stream, float* stage_ms,
                                           int32_t* stage_launches);

/* ---- Frozen-base backward --------------------------------------------------
 * The GEMM backward that bypasses the base weight gradient (Orbit
 * announcement, 技术细节): gradients for the layer inputs and the adapter only.
 * Its two GEMMs contract over the weights' output dimension, so they read a
 * transposed copy of the frozen weights, made once per base. */

/* Bytes of the transposed copy: W13^T [E][H][2I] and W2^T [E][I][H] in the
 * format's codes (INT4 / E2M1 nibbles, E4M3 bytes), stored in tiles of 16
 * rows x 128 codes as MOE_WL_KBLOCKED describes, plus scales (INT4, MXFP4,
 * NVFP4: one fp16 per group scale; FP8: the fp32 block scales transposed); 0 if the
 * layer is not supported by the backward (I multiple of 256; FP8 H and 2I at
 * most 8192). */
size_t moe_backward_weights_bytes(const moe_layer* layer);

/* Writes the transposed copy of (qweights, scales) into bwd_weights (device,
 * caller-owned, >= moe_backward_weights_bytes).  Codes are bit-identical
 * re-layouts; INT4 scales are converted to fp16 (exact for bf16 scales in
 * [2^-17, 8188]), MXFP4
 * scales to fp16 2^(e-127) (exact within fp16's range), NVFP4 E4M3 scales
 * to fp16 (exact), FP8 block scales are transposed.  NVFP4's fp32
 * second-level scales are not copied: moe_expert_backward reads them from
 * its moe_scales (g13 / g2 required there, 4-byte aligned). */
moe_status moe_prepare_backward_weights(const moe_layer* layer, const moe_qweights* qweights,
                                        const moe_scales* scales, void* bwd_weights, size_t bwd_bytes,
                                        void* stream);

/* Workspace bytes of moe_expert_backward (routing, recomputed gate/up
 * pre-activations fp32 [R][2I], their gradients fp16 [R][2I], dx' fp32
 * [R][H] (twice with an adapter), the fp16 copy of d_out, and for a shared
 * adapter the per-expert gradient partials fp32 [E][H/32][32][32]). */
size_t moe_backward_workspace_bytes(const moe_layer* layer, int32_t chunk_experts);

/* Backward of moe_expert_forward for given d_out = dL/dout [T][H] bf16:
 *   d_x      [T][H] bf16    dL/dx
 *   d_logits [T][E] fp32    dL/dlogits: w_tj (g_tj - sum_i w_ti g_ti) for the
 *                           selected experts, g_tj = <d_out_t, y_tj>; 0 elsewhere
 *   d_adapter fp32, shaped like the adapter, dL/dR (a shared R, stride 0,
 *                           gets the sum over all experts, added in ascending
 *                           active-expert order); NULL exactly when adapter is NULL
 * No gradient is formed for W13 or W2.  The forward is recomputed per chunk
 * (routing, gate/up pre-activations); per permuted row (t, j) of expert e:
 * u = d_out_t W2, dh = w_tj u, da = dh b silu'(a), db = dh silu(a),
 * dx' = da Wg + db Wu, dR_e += x_t^T dx' (32x32 diagonal blocks),
 * dx_tj = dx' R_e^T, d_x_t = sum_j dx_tj.  Activation quantizers of the
 * FP8 / MXFP4 formats pass gradients straight through; the router term uses
 * h as the forward quantized it.  GEMM operands are fp16 (INT4 and E2M1
 * weights times their scales exactly, NVFP4's second-level scale applied to
 * the fp32 accumulators, E4M3 times the block scale rounded once; d_out and the SwiGLU gradients rounded to fp16, so their magnitudes
 * must stay below 65504), accumulation fp32.
 * bwd_weights: from moe_prepare_backward_weights for the same weights.
 * Unsupported layers return MOE_ERR_UNSUPPORTED; the rest as moe_expert_forward.
 * Stream-ordered, no host synchronisation, nothing allocated, unless
 * stage_ms and stage_launches (HOST arrays of MOE_NUM_STAGES, both or
 * neither) are given: then per-stage event times are filled as by
 * moe_expert_forward_timed and the call synchronises the stream.  Stages:
 * ROUTE, PERMUTE; ACT = GEMM inputs (x or x R_e, d_out as fp16); GEMM1 =
 * gate/up recompute launches; GEMM2 = backward GEMM launches (chunk c's
 * u items with chunk c-1's dx' items); COMBINE = adapter backward,
 * un-permute sum and router gradient. */
moe_status moe_expert_backward(const moe_layer* layer, const void* x_bf16, const float* logits,
                               const moe_qweights* qweights, const moe_scales* scales, const void* bwd_weights,
                               const void* adapter_bf16, const void* d_out_bf16, int32_t chunk_experts,
                               void* d_x_bf16, float* d_logits, float* d_adapter, void* ws, size_t ws_bytes,
                               void* stream, float* stage_ms, int32_t* stage_launches);

/* The GEMM1 input quantizer of the layer's weight format applied to x, one
 * row per token (what moe_expert_forward feeds its first grouped GEMM when no
 * adapter is given), written to caller buffers:
 *   FP8 (NeMo RL FP8 post, Table 1, input activations): codes [T][H] E4M3FN,
 *     scales fp32 [T][H/128]: s = amax/448 (1 for an all-zero block),
 *     q = RNE-saturate(v/s), both quotients correctly rounded in fp32;
 *   FP8_POW2: as FP8 with s the smallest power of two >= amax/448;
 *   MXFP4: codes [T][H] E4M3FN, scales [T][H/32] E8M0 bytes: shared exponent
 *     X = floor(log2 amax) - 8 (0 for an all-zero block, clamped to
 *     [-127, 127]), q = RNE-saturate(v * 2^-X).
 * INT4 and NVFP4 layers take 16-bit activations and have no quantizer:
 * MOE_ERR_UNSUPPORTED.  x, codes: 16-byte aligned; scales: 4-byte aligned.
 * Stream-ordered, no host synchronisation. */
moe_status moe_quantize_activations(const moe_layer* layer, const void* x_bf16, void* codes, void* scales,
                                    void* stream);

/* Weighted combine on its own: out[t] = sum_{j<k} topk_w[t][j] *
 * y_perm[row_of[t*k+j]], fp32 sum in ascending j, RNE to bf16.  y_perm:
 * [T*k][H] bf16.  Atomic-free and deterministic. */
moe_status moe_combine(const moe_layer* layer, const void* y_perm_bf16, const float* topk_w,
                       const int32_t* row_of, void* out_bf16, void* stream);

/* Workspace bytes moe_lm_head_logprob needs: T*ceil(V/128)*2 fp32
 * log-softmax statistics (maximum and sum of exponentials per token and
 * block of 128 vocabulary rows) and T fp32 target logits, each 256-byte
 * aligned. */
size_t moe_lm_head_workspace_bytes(int32_t T, int32_t V);

/* Log-prob of target tokens under an LM head (the rollout log-probs whose
 * train/rollout agreement the NeMo RL FP8 post measures with its
 * token-mult-prob-error):  z = h / sqrt(mean(h^2) + 1e-6) (a final
 * parameter-free RMSNorm), logits = z W_lm^T (fp32 accumulation),
 * logprob[t] = logits[t][y_t] - logsumexp_v logits[t][v].
 * h: [T][H] bf16; w_lm: [V][H] bf16; targets: [T] int32 in [0, V);
 * logprob: [T] fp32.  H multiple of 128, T <= 4096. */
moe_status moe_lm_head_logprob(int32_t T, int32_t H, int32_t V, const void* h_bf16, const void* w_lm_bf16,
                               const int32_t* targets, float* logprob, void* ws, size_t ws_bytes,
                               void* stream);

/* ---- Allocation-free forward -------------------------------------------
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same computation, arguments (minus ws / ws_bytes) and result
 * as moe_expert_forward; the workspace is instead a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, reserved when
 * the library is loaded on that GPU and held until the process ends.  Layers
 * whose moe_workspace_bytes() exceeds it (e.g. more than a few thousand
 * tokens at hidden 7168) return MOE_ERR_WORKSPACE_TOO_SMALL with nothing
 * enqueued.  The call allocates nothing (no hipMalloc, no library
 * allocation); the first call on a device looks up that device's array
 * address once.  The stream must belong to the current device.  Every call on
 * one GPU uses the same array, whose contents persist between calls and are
 * overwritten by each call: calls that overlap on one GPU (other streams,
 * other host threads) race and must be serialised by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_expert_forward_noalloc(const moe_layer* layer, const void* x_bf16, const float* logits,
                                      const moe_qweights* qweights, const moe_scales* scales,
                                      const void* adapter_bf16, int32_t chunk_experts, void* out_bf16,
                                      void* stream);

/* Static description of a status code (never NULL). */
const char* moe_status_str(moe_status status);

/* MOE_LP_ABI_VERSION of the built library. */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LP_H */
