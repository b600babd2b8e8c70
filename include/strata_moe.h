/*
 * strata_moe.h — C ABI of the routed Mixture-of-Experts expert layer for MI355X (gfx950).
 *
 * The layer: each token picks k of E experts from its router logits, every picked expert runs a
 * SwiGLU feed-forward network on block-quantized 2- or 3-bit weights, and the token's output is
 * the router-weighted sum of its experts' outputs.
 *
 * Sources.  The pages describe a model whose layers each hold 512 experts with 10 active per
 * token over 48 layers ("Strata vs Llama.cpp vs vLLM", transcript at 08:23; "Local AI Is Now 6x
 * Faster on Your PC", key technological idea).  They name the expert matrix multiply as the
 * heaviest computation and say it dequantizes low-bit blocks during the multiply ("Two-Day Port,
 * 8x Faster Prefill: Strata Engine Benchmarked", Where Strata Is Fast).  They say k-quants go down
 * to two or three bits per weight and are dequantized on the fly ("Strata vs Llama.cpp vs vLLM",
 * transcript at 04:12).  The pages print neither the router formula, the FFN form, nor any bit
 * layout; the definitions below (softmax top-k routing, SwiGLU, the Q2/Q3 block formats) are this
 * library's specification and are stated in full where each call is declared.
 *
 * Conventions that hold for every entry point:
 *  - Every pointer argument that is not marked "host" is a device pointer (hipMalloc'd memory,
 *    e.g. a torch tensor's data_ptr()).  The caller allocates and owns all buffers; the library
 *    never allocates, frees or synchronises.  Scratch memory comes from a caller-provided
 *    workspace whose size strata_moe_workspace_bytes() returns.
 *  - Device pointers must be 16-byte aligned (128-bit loads and stores).
 *  - All work is enqueued asynchronously on `stream` (NULL = the null stream).  The return code
 *    is synchronous: arguments are validated before any HIP call, and on any error nothing has
 *    been enqueued.  STRATA_ERR_HIP means a launch itself failed.  Device-side faults surface at
 *    the caller's next synchronisation.
 *  - T = 0 is a no-op that returns STRATA_OK.
 *  - The library holds no global mutable state; calls on different streams with disjoint
 *    outputs and workspaces may run concurrently.
 *  - Non-finite logits, activations or scales are outside the contract (not checked).
 *  - Results are deterministic: the same inputs give bit-identical outputs on every call
 *    (no floating-point atomics anywhere).
 */
#ifndef STRATA_MOE_H
#define STRATA_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STRATA_OK = 0,
  STRATA_ERR_INVALID_ARGUMENT = 1,   /* null or misaligned pointer, non-positive size, k > E ... */
  STRATA_ERR_UNSUPPORTED = 2,        /* well-formed but outside what the kernels handle        */
  STRATA_ERR_WORKSPACE_TOO_SMALL = 3,
  STRATA_ERR_HIP = 4,                /* a kernel launch failed                                  */
  /* not a status: makes the type span every non-negative int32, so that an unknown code handed
   * to strata_status_string is a valid value of it in C++ as well as in C */
  STRATA_STATUS_MAX_ENUM_ = 0x7FFFFFFF
} strata_status;

/*
 * Block-quantized weight formats.  A block is 32 consecutive weights along the reduction
 * dimension of a matrix row, with one fp16 (IEEE binary16) scale d per block.
 *
 * STRATA_Q2_B32: 2-bit codes q in {0..3}; w = d * (q - 1.5).  A block's codes take 8 bytes:
 *   weight i (0..31) sits in bits [2*(i%16), 2*(i%16)+1] of little-endian uint32 word i/16,
 *   i.e. byte i/4, bits [2*(i%4), 2*(i%4)+1].
 * STRATA_Q3_B32: 3-bit codes q in {0..7}; w = d * (q - 3.5).  A block's codes take 12 bytes
 *   read as one 96-bit little-endian integer; weight i sits in bits [3*i, 3*i+2] (codes may
 *   straddle byte and word edges).
 *
 * Row-major layout.  A matrix with R rows and reduction length K (K a multiple of 32) is two
 * arrays (structure of arrays):
 *   codes  [R][K/32][cb bytes]      (cb = 8 for Q2, 12 for Q3)
 *   scales [R][K/32] fp16
 * so w[r][c] = scale[r][c/32] * (code of weight c%32 in block [r][c/32] - offset).
 *
 * Tiled layout (what the compute entry points read).  R a multiple of 4 and K of 64; the matrix
 * is cut into tiles of 4 rows x 64 reduction indices (two blocks per row), ordered row-group
 * major:
 *   codes  [R/4][K/64][4][2][cb bytes]
 *   scales [R/4][K/64][4][2] fp16
 * i.e. block b of row r sits at tile (r/4, b/2), tile row r%4, slot b%2.  The same bytes as the
 * row-major arrays, reordered so that a 4-row group's consecutive 64-index stages are contiguous
 * and one stage of 64 rows is 16 contiguous pieces.
 * strata_moe_pack_matrix converts row-major -> tiled on the device.
 */
typedef enum {
  STRATA_Q2_B32 = 2,
  STRATA_Q3_B32 = 3
} strata_qformat;

/*
 * Per-expert range statistics of a layer's weights (device array [E], written once by
 * strata_moe_weight_stats).  The prefill path feeds fp16 operands to the matrix cores; these
 * numbers let it place every operand inside fp16's range exactly, by powers of two, whatever
 * the block scales and the activations' magnitude:
 *   shift_gate, shift_up, shift_down: the exponent s of each matrix such that its largest
 *     |d| * max|q - c0| times 2^s lies in [2^14, 2^15), capped at 15 for STRATA_Q2_B32; the GEMM
 *     uses fp16(d * 2^s * (q - c0)) and takes 2^-s back out of its fp32 sums (0 for an all-zero
 *     matrix);
 *   norm_gate_up: an upper bound of (max over rows of the 2-norm of the shifted gate rows) times
 *     (the same for the up rows).  With x's own 2-norm it bounds |SiLU(g) * u| by Cauchy-Schwarz,
 *     and so fixes a per-row power of two that keeps the intermediate a below 2^15 in fp16.
 * The decode path reads the scales directly and does not use these.
 */
typedef struct strata_moe_expert_stats {
  int32_t shift_gate;
  int32_t shift_up;
  int32_t shift_down;
  float norm_gate_up;
} strata_moe_expert_stats;

/*
 * One layer's expert weights, all device pointers, expert-major, each matrix in the tiled layout:
 *   gate W_g and up W_u: per expert an [I][H] matrix (rows = intermediate features, reduction
 *     along H): codes [E][I/4][H/64][4][2][cb], scales [E][I/4][H/64][4][2];
 *   down W_d: per expert an [H][I] matrix (rows = hidden features, reduction along I):
 *     codes [E][H/4][I/64][4][2][cb], scales [E][H/4][I/64][4][2];
 * with cb = 8 (Q2) or 12 (Q3).  Expert e's arrays start at e times the per-expert size (the E
 * matrices of one kind are also one tiled matrix of E*R rows).
 * Field order: format and sizes, then gate and up codes, gate and up scales, down codes, down
 * scales (byte offsets on LP64: 0, 4, 8, 12, 16, 24, 32, 40, 48, 56), then stats (offset 64):
 * the range statistics above, required by the prefill path (strata_moe_expert_ffn, and
 * strata_moe_layer and its callers when they take it) and ignored by the decode path (may be
 * NULL there).
 */
typedef struct strata_moe_weights {
  int32_t fmt;          /* strata_qformat */
  int32_t num_experts;  /* E: 1..1024 */
  int32_t hidden;       /* H: multiple of 256 */
  int32_t inter;        /* I: multiple of 128 */
  const void* gate_codes;
  const void* up_codes;
  const uint16_t* gate_scales;
  const uint16_t* up_scales;
  const void* down_codes;
  const uint16_t* down_scales;
  const strata_moe_expert_stats* stats;
} strata_moe_weights;

/*
 * Range statistics of w's tiled weights (see strata_moe_expert_stats): a one-time load step
 * after strata_moe_pack_matrix, like the repack itself.  w->stats is not read.
 *   stats  device array [w->num_experts] (written)
 * Errors as for the compute calls (w's sizes and pointers are validated).
 */
strata_status strata_moe_weight_stats(const strata_moe_weights* w, strata_moe_expert_stats* stats,
                                      hipStream_t stream);

/*
 * Router: per-token top-k selection and weights.
 * The pages say each token is routed to 10 of a layer's 512 experts and that the routers run on
 * the GPU ("Strata vs Llama.cpp vs vLLM", transcript 08:23 and 09:28; "Strata - the details",
 * How it works / memory tiers); they give no formula.  This library's definition: softmax over
 * all E logits, keep the k largest, renormalise.  Selection is made on the fp32 logits
 * themselves (softmax is monotone); expert a beats expert b iff l_a > l_b, or l_a == l_b and
 * a < b.  Slot j (0..k-1) holds the j-th pick (descending logit).  The renormalised weights are
 * w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k picks (the full softmax denominator
 * cancels).
 *
 *   logits   fp32 [T][E] row-major (read)
 *   topk_ids int32 [T][k] (written)
 *   topk_w   fp32 [T][k] (written)
 * Limits: 1 <= k <= min(E, 16), 1 <= E <= 1024.
 */
strata_status strata_moe_route(const float* logits, int32_t T, int32_t E, int32_t k,
                               int32_t* topk_ids, float* topk_w, hipStream_t stream);

/*
 * Permute: group the S = T*k (token, slot) pairs by expert with a stable counting sort.
 * Implied by per-expert matrix multiplies ("Two-Day Port, 8x Faster Prefill: Strata Engine
 * Benchmarked", Where Strata Is Fast); the pages give no algorithm.  Slot s = t*k + j.
 *   counts      int32 [E]    number of slots routed to expert e
 *   offsets     int32 [E+1]  exclusive prefix sum of counts; offsets[E] = S
 *   sorted_slot int32 [S]    position p -> slot; expert e's segment is
 *                            [offsets[e], offsets[e+1]) in ascending slot order
 *   slot_pos    int32 [S]    inverse: slot -> position
 * Workspace: at least strata_moe_permute_workspace_bytes(T, E, k).
 * Limits: as strata_moe_route; S < 2^31.
 */
strata_status strata_moe_permute(const int32_t* topk_ids, int32_t T, int32_t E, int32_t k,
                                 int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                                 int32_t* slot_pos, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * Expert FFN (prefill path): for every expert e and every slot s in its segment (token t =
 * s / k), with x the token's activations:
 *   g = W_g x,  u = W_u x,  a = SiLU(g) * u  (SiLU(z) = z / (1 + exp(-z))),  out = W_d a.
 * The pages call the expert matrix multiply the heaviest computation and describe dequantizing
 * the low-bit blocks during the multiply ("Two-Day Port, 8x Faster Prefill: Strata Engine
 * Benchmarked", Where Strata Is Fast); the gate/up/SiLU-mul/down form is this library's
 * definition.  Precision: the products run on fp16 matrix cores with fp32 accumulation, every
 * operand brought into fp16's range by exact powers of two that the fp32 epilogues take back out:
 *  - x: each token row is scaled so that its largest |x| lies in [2^14, 2^15); the bf16 values
 *    then convert to fp16 exactly (down to 2^-31 of the row's largest);
 *  - weights: each dequantized weight is fp16(d * 2^s * (q - c0)), one rounding, with the
 *    matrix's shift s from w->stats (no overflow for any finite scale; blocks within 2^28 of the
 *    matrix's largest stay normal);
 *  - a = SiLU(g) * u: rounded once to fp16 after scaling by a per-row power of two that puts the
 *    row's Cauchy-Schwarz bound |x| * max|W_g row| * max|W_u row| just below 2^15;
 *  - out is rounded to bf16.
 * The result stays within 5e-3 per-row relative L2 of the exact (fp64) layer for activation
 * rows whose largest |x| lies in [2^-100, 2^100] and any finite block scales (outside that the
 * token scaling stops at 2^+-113 and tiny rows lose precision); w->stats must not be NULL.
 *
 *   x           bf16 [T][H] (uint16 bit patterns)
 *   offsets, sorted_slot  as produced by strata_moe_permute for this (T, k, E)
 *   expert_out  bf16 [T*k][H], row s = slot s (unweighted expert output), written
 * Workspace: at least strata_moe_workspace_bytes(T, E, k, H, I).
 * Limits: w->hidden a multiple of 256, w->inter a multiple of 128; E, k as strata_moe_route.
 */
strata_status strata_moe_expert_ffn(const strata_moe_weights* w, const uint16_t* x, int32_t T,
                                    int32_t k, const int32_t* offsets,
                                    const int32_t* sorted_slot, uint16_t* expert_out,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Combine: y[t] = sum_{j = 0..k-1, ascending} topk_w[t][j] * expert_out[t*k + j]   (fp32),
 * and with accumulate != 0, y[t] += that sum instead (the residual add of a layer stack).
 * The pages say each token's output comes from the 10 experts it is routed to ("Strata vs
 * Llama.cpp vs vLLM", transcript at 08:23; "Local AI Is Now 6x Faster on Your PC", key
 * technological idea) without spelling the combination out; the router-weighted sum is this
 * library's definition.
 *   expert_out bf16 [T*k][H], topk_w fp32 [T][k], y fp32 [T][H].
 */
strata_status strata_moe_combine(const uint16_t* expert_out, const float* topk_w, int32_t T,
                                 int32_t k, int32_t H, float* y, int32_t accumulate,
                                 hipStream_t stream);

/*
 * Decode / verify step for T <= 8 tokens (the pages' multi-token-prediction check of up to 3
 * drafted tokens plus one: "Strata - the details", How it works / speculation).  Computes the
 * same function as route + permute + expert_ffn + combine, with a bandwidth-bound path: every
 * touched expert's weights are streamed once and applied to all tokens that picked it.
 * Precision: weights and x enter exactly (bf16 dot products of the codes, fp32 accumulation, the
 * fp16 block scale applied in fp32); a is rounded to bf16; the expert outputs and y stay fp32.
 * The combine sums the k outputs of a token in slot order, so the result is deterministic.
 *   x bf16 [T][H], logits fp32 [T][E], y fp32 [T][H] (overwritten, or += with accumulate)
 *   opt_topk_ids int32 [T][k], opt_topk_w fp32 [T][k]: written when not NULL.
 * Workspace: at least strata_moe_workspace_bytes(T, E, k, H, I).
 * Limits: 1 <= T <= 8, T*k <= 128, hidden and inter at most 4096, and the activations staged
 * in LDS must fit: 19/8 * T * hidden + 4 * E <= 147456 and 19/8 * T * k * inter <= 147456 (bytes);
 * STRATA_ERR_UNSUPPORTED otherwise.  Others as strata_moe_expert_ffn.
 */
strata_status strata_moe_decode(const strata_moe_weights* w, const uint16_t* x,
                                const float* logits, int32_t T, int32_t k, float* y,
                                int32_t accumulate, int32_t* opt_topk_ids, float* opt_topk_w,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * strata_moe_decode without a workspace argument, for callers that cannot allocate device memory
 * or pass one: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same computation, kernels and results as strata_moe_decode.  The scratch memory is
 * a fixed device array inside the library, strata_moe_decode_static_max_bytes() bytes on each GPU
 * it runs on (held until the process ends); the call allocates and frees nothing.  Every call on
 * one GPU uses that GPU's array, so calls that overlap on one GPU (different streams, or
 * different threads without ordering) race and must not be made; nothing in it needs to start
 * zeroed.  Arguments and limits as strata_moe_decode.  The array holds 128 KiB, enough for every
 * shape within those limits (the largest needs 126,720 bytes); a shape whose decode workspace did
 * not fit would return STRATA_ERR_WORKSPACE_TOO_SMALL before any HIP call.
 */
strata_status strata_moe_decode_static(const strata_moe_weights* w, const uint16_t* x,
                                       const float* logits, int32_t T, int32_t k, float* y,
                                       int32_t accumulate, int32_t* opt_topk_ids,
                                       float* opt_topk_w, hipStream_t stream);
size_t strata_moe_decode_static_max_bytes(void);

/*
 * One-call layer: y (=, or += with accumulate) MoE(x): route each token to k of the E experts,
 * run the experts it picked, sum their outputs weighted by the router.  The pages' layer routes
 * each token to 10 of 512 experts ("Strata vs Llama.cpp vs vLLM", transcript at 08:23; "Two-Day
 * Port, 8x Faster Prefill: Strata Engine Benchmarked", Where Strata Is Fast); the steps and their
 * definitions are those of strata_moe_route, strata_moe_permute, strata_moe_expert_ffn and
 * strata_moe_combine.
 * T <= 8 runs strata_moe_decode's path when the shape is within its limits.  9 <= T <= 32 runs
 * the same decode path on consecutive slices of at most 8 tokens (the layer's tokens are
 * independent; with few rows per expert, streaming each touched expert once per slice is faster
 * than the grouped GEMMs).  Otherwise route -> permute -> expert_ffn -> combine.
 * Each opt_* pointer may be NULL; when given it receives that intermediate in the layout of the
 * staged calls: opt_topk_ids int32 [T][k], opt_topk_w fp32 [T][k], opt_counts int32 [E],
 * opt_offsets int32 [E+1], opt_sorted_slot int32 [T*k].  On the decode paths the permutation is
 * produced, when asked for, by one extra counting-sort launch over the routing result.
 * Workspace: at least strata_moe_workspace_bytes(T, E, k, H, I).
 */
strata_status strata_moe_layer(const strata_moe_weights* w, const uint16_t* x, const float* logits,
                               int32_t T, int32_t k, float* y, int32_t accumulate,
                               int32_t* opt_topk_ids, float* opt_topk_w, int32_t* opt_counts,
                               int32_t* opt_offsets, int32_t* opt_sorted_slot, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * One layer of a stack with a residual stream: h <- h + MoE(RMSNorm(h)), with
 * RMSNorm(h)[t] = bf16_RNE(h[t] / sqrt(mean_i h[t][i]^2 + eps)) (unit gain, as strata_moe_rmsnorm).
 * The pages' model runs 48 such MoE layers ("Strata vs Llama.cpp vs vLLM", transcript at 08:23);
 * the pre-norm residual form is this library's definition.  For T <= 8 (decode limits as
 * strata_moe_decode) the normalisation is formed inside the decode path's first kernel (no separate
 * launch); otherwise strata_moe_rmsnorm into the workspace, then strata_moe_layer accumulating into h.
 *   h      fp32 [T][H] (read and written)
 *   logits fp32 [T][E] (read)
 * Workspace: at least strata_moe_residual_workspace_bytes(T, E, k, H, I).  eps >= 0.
 */
strata_status strata_moe_layer_residual(const strata_moe_weights* w, float* h, const float* logits,
                                        int32_t T, int32_t k, float eps, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);

/*
 * Weight repack, row-major -> tiled (see the layouts above), for n_mat matrices of rows x K
 * stored back to back (e.g. all E gate matrices: n_mat = E, rows = I, K = H).  A one-time
 * load step; the compute entry points read only the tiled layout.
 *   codes, scales              row-major arrays (read)
 *   tiled_codes, tiled_scales  same sizes, tiled (written); must not overlap the inputs
 * Limits: rows a multiple of 4 and K a multiple of 64 (STRATA_ERR_UNSUPPORTED otherwise).
 */
strata_status strata_moe_pack_matrix(int32_t fmt, int32_t n_mat, int32_t rows, int32_t K,
                                    const void* codes, const uint16_t* scales, void* tiled_codes,
                                    uint16_t* tiled_scales, hipStream_t stream);

/*
 * RMSNorm for a layer stack: x[t] = bf16_RNE(h[t] / sqrt(mean_i h[t][i]^2 + eps)), unit gain.
 *   h fp32 [T][H] (read), x bf16 [T][H] (written).  H a multiple of 4.
 */
strata_status strata_moe_rmsnorm(const float* h, int32_t T, int32_t H, float eps, uint16_t* x,
                                 hipStream_t stream);

/*
 * Router projection: logits[t][e] = sum_h x[t][h] * w_router[e][h], fp32.  The pages keep the
 * routers on the GPU with the experts ("Strata - the details", How it works / memory tiers;
 * "Strata vs Llama.cpp vs vLLM", transcript at 09:28) but give no formula; a dense linear map of
 * the normalised hidden state to one logit per expert is this library's definition.  The
 * logits feed strata_moe_route / strata_moe_layer.
 *   x        bf16 [T][H] (read), the layer input after RMSNorm
 *   w_router bf16 [E][H] (read), row-major
 *   logits   fp32 [T][E] (written)
 * Precision: bf16 products are exact in fp32; sums are accumulated in fp32 (matrix cores for
 * T > 8, dot-product instructions for T <= 8), so |logits - exact| <= H * 2^-24 / (1 - H * 2^-24)
 * * sum_h |x[t][h] w_router[e][h]|.
 * Limits: H a multiple of 64 (STRATA_ERR_UNSUPPORTED otherwise); E >= 1.
 */
strata_status strata_moe_router_logits(const uint16_t* x, const uint16_t* w_router, int32_t T,
                                       int32_t H, int32_t E, float* logits, hipStream_t stream);

/*
 * Shared expert, a dense SwiGLU FFN applied to every token: a = bf16_RNE(SiLU(x W_sg^T) *
 * (x W_su^T)), out = a W_sd^T, y = out (or y += out with accumulate != 0).  The pages list shared
 * experts among what stays on the GPU ("Strata - the details", How it works / memory tiers;
 * "Strata vs Llama.cpp vs vLLM", transcript at 09:28); its form, the routed experts' SwiGLU with
 * dense weights and no router scale, is this library's definition.
 *   x          bf16 [T][H] (read)
 *   w_gate     bf16 [I][H], w_up bf16 [I][H], w_down bf16 [H][I] (read), row-major
 *   y          fp32 [T][H] (written or accumulated)
 * Workspace: at least strata_moe_shared_workspace_bytes(T, I) (holds a).
 * Precision: fp32 accumulation of exact bf16 products; a rounded to bf16 once.
 * Limits: H and I multiples of 64 (STRATA_ERR_UNSUPPORTED otherwise).
 */
strata_status strata_moe_shared_expert(const uint16_t* x, const uint16_t* w_gate,
                                       const uint16_t* w_up, const uint16_t* w_down, int32_t T,
                                       int32_t H, int32_t I, float* y, int32_t accumulate,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/*
 * One whole MoE block step: logits = x W_r^T (written, as strata_moe_router_logits), the routed
 * layer on those logits (as strata_moe_layer) and the shared expert (as strata_moe_shared_expert),
 * y = routed + shared (y += both with accumulate != 0).  The pages keep the routers and the shared
 * experts on the GPU beside the routed experts ("Strata vs Llama.cpp vs vLLM", transcript at 09:28;
 * "Strata - the details", How it works / memory tiers); the block's composition is this library's
 * definition.  For T <= 8 within the decode limits (strata_moe_decode) it is three launches: the
 * router and the shared gate/up projection in one GEMV, then the decode kernels, the first of
 * which also applies the shared down projection while its routing waves route; otherwise the
 * three entry points above in turn.
 *   x        bf16 [T][H] (read)
 *   w_router bf16 [E][H]; w_sgate, w_sup bf16 [Is][H]; w_sdown bf16 [H][Is] (read), row-major
 *   logits   fp32 [T][E] (written)
 *   y        fp32 [T][H] (written or accumulated)
 * Workspace: at least strata_moe_block_workspace_bytes(T, E, k, H, I, Is).
 * Limits: those of strata_moe_layer and strata_moe_shared_expert (Is a multiple of 64).
 */
strata_status strata_moe_block(const strata_moe_weights* w, const uint16_t* x, int32_t T, int32_t k,
                               const uint16_t* w_router, const uint16_t* w_sgate,
                               const uint16_t* w_sup, const uint16_t* w_sdown, int32_t Is,
                               float* logits, float* y, int32_t accumulate, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);
size_t strata_moe_block_workspace_bytes(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I,
                                        int32_t Is);

/*
 * Expert usage statistics.  The pages' engine keeps a running distribution of how often each
 * expert is used and keeps the most-used experts nearest the compute (video transcript on
 * unbiasedbob.com, 7:47 to 7:58; "Strata - the details", How it works / memory tiers).  This
 * library's statistic: usage[e] += the number of (token, slot) pairs of topk_ids routed to e
 * (ids outside [0, E) are ignored), in 64-bit integers, so it accumulates exactly over calls;
 * the caller zeroes usage to start a new window.
 *   topk_ids int32 [T][k] (read; e.g. the opt_topk_ids output of strata_moe_layer)
 *   usage    uint64 [E] (read and written)
 * Limits: E <= 1024 (STRATA_ERR_UNSUPPORTED otherwise).
 */
strata_status strata_moe_usage_update(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                                     uint64_t* usage, hipStream_t stream);

/*
 * Hotness order of the experts: order[r] = the expert of rank r by usage, most used first, equal
 * usage broken by the lower expert index (a permutation of 0 .. E-1).
 *   usage uint64 [E] (read), order int32 [E] (written).  E <= 1024.
 */
strata_status strata_moe_usage_rank(const uint64_t* usage, int32_t E, int32_t* order,
                                   hipStream_t stream);

/* Workspace sizes in bytes (host functions).  0 for a shape every compute call rejects: T < 0,
 * E outside 1..1024, k outside 1..min(E, 16), T * k above 2^30 - 1, H or I below 1. */
size_t strata_moe_permute_workspace_bytes(int32_t T, int32_t E, int32_t k);
size_t strata_moe_workspace_bytes(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I);
size_t strata_moe_shared_workspace_bytes(int32_t T, int32_t I);
size_t strata_moe_residual_workspace_bytes(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I);

/* Static string for a status code (host function; never NULL). */
const char* strata_status_string(strata_status status);

#ifdef __cplusplus
}
#endif

#endif /* STRATA_MOE_H */
