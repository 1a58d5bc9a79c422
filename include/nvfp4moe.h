/*
 * nvfp4moe.h - C ABI of the MI355X (gfx950) NVFP4 mixture-of-experts expert
 * pipeline.
 *
 * The pipeline is: quantise the layer input to NVFP4, route each token to its
 * top-k experts and group the (token, expert) rows by expert, run the first
 * grouped GEMM against the stacked gate_up weights, apply SiLU(gate) * up and
 * re-quantise the intermediate to NVFP4, run the second grouped GEMM against
 * the down weights, and combine each token's k expert outputs with the routing
 * weights.  This is the expert pipeline planned on the page "Current Bug: vLLM
 * produces empty/garbage output" (revision e8b289e, section "Revised Plan: Our
 * Own NVFP4 Kernels", Phase 1), with 384 experts and top-6 routing in the
 * full model ("CURRENT_BUG.md - DeepSeek-V4 Blackwell NVFP4", section
 * "Architecture Notes").  The shared expert is the same pipeline with one
 * group and no routing, and the MLA projections are one-group GEMMs.
 *
 * NVFP4 tensor layout (row-major, C columns, C a multiple of 16):
 *   codes  uint8 [rows, C/2]   E2M1 codes, element 2i in the LOW nibble of
 *                              byte i, element 2i+1 in the high nibble;
 *                              bit 3 of a code is the sign, bits 0-2 index
 *                              the magnitudes {0,0.5,1,1.5,2,3,4,6}.
 *   scales uint8 [rows, C/16]  one E4M3 (FN: bias 7, max 448) code per 16
 *                              consecutive elements of a row, no swizzle.
 *   gs     float32             one global scale per tensor in the
 *                              DEQUANTISATION direction:
 *                              value = gs * e4m3(scale) * e2m1(code).
 * The direction matters: the page revision a51edd2 ("What the quant method
 * does") shows a scale used as its own inverse blowing activations up to
 * NaN.  Here quantisation divides by gs and saturates (block scale 448, code
 * +-6) instead of overflowing.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is DEVICE memory owned by the caller unless the
 *     comment says "host".  The library never allocates, frees or
 *     synchronises; all work is enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream).  Device-side faults surface at the caller's next
 *     synchronisation.
 *   - Arguments are validated on the host before any HIP call; a failing
 *     check returns a non-zero status and launches nothing.
 *     nvfp4_last_error() then describes the failure (thread-local string).
 *   - Index arrays produced on the device (row indices, group offsets) are
 *     not trusted: kernels clamp them so that no access leaves the buffers
 *     whose sizes were passed in; out-of-range entries give unspecified
 *     values, never out-of-bounds accesses.
 *   - Inputs must be finite; NaN/Inf inputs give unspecified codes.
 *   - Calls are deterministic: the same inputs give bit-identical outputs.
 *   - Setting the environment variable NVFP4MOE_SYNC_CHECK=1 makes every entry
 *     point synchronise its stream after launching and report kernel faults
 *     as NVFP4_EHIP (a debugging aid; off by default).
 */
#ifndef NVFP4MOE_H
#define NVFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define NVFP4_OK 0
#define NVFP4_EINVAL 1      /* null pointer, unknown enum value, negative size */
#define NVFP4_ESHAPE 2      /* a size constraint does not hold */
#define NVFP4_EALIGN 3      /* a pointer is not aligned as required */
#define NVFP4_EHIP 4        /* the HIP runtime reported an error */

/* Element types of float tensors crossing the boundary. */
#define NVFP4_DTYPE_F32 0
#define NVFP4_DTYPE_BF16 1

/* Layouts of the weight operand of nvfp4_grouped_gemm. */
#define NVFP4_LAYOUT_ROWS 0   /* codes [G, N, K/2] and scales [G, N, K/16], row-major */
#define NVFP4_LAYOUT_TILED 1  /* one buffer written by nvfp4_prepare_weights */

/* Upper limits checked by the entry points. */
#define NVFP4_MAX_EXPERTS 1024
#define NVFP4_MAX_TOPK 16
#define NVFP4_MAX_SEGMENTS 4

/* Message describing the last failing call on this thread ("" if none). */
const char* nvfp4_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int32_t nvfp4_version(void);

/*
 * nvfp4_quantize - quantise a float tensor to NVFP4 with a given global
 * scale.
 *   x        [rows, ld_x] of x_dtype (F32 or BF16); columns [0, cols) are
 *            quantised.  16-byte aligned, ld_x*elem_size a multiple of 16.
 *   gs       device pointer to ONE float32, the global scale (dequantisation
 *            direction, > 0).
 *   codes    out [rows, cols/2], scales out [rows, cols/16], both dense.
 *   dq       out [rows, cols] f16 (uint16 storage, 16-byte aligned) or NULL:
 *            the dequantised values e2m1(code) * e4m3(scale) WITHOUT the
 *            global scale.  They are exact in f16 (at most five significant
 *            bits, magnitudes in [2^-10, 2688]).  nvfp4_grouped_gemm can read
 *            A in this form (a_dq) instead of decoding it itself.
 * Per 16-element block (each step one IEEE float32 operation, no fused
 * multiply-add): bamax = max|x_i|; s = bamax / (6*gs); sq = E4M3(s), rounded
 * to nearest-even and saturated at 448; sf = value(sq).  If sf == 0 every
 * code of the block is 0x0.  Otherwise r = 1/(sf*gs) and code_i = sign bit of
 * x_i, plus the E2M1 magnitude nearest to |x_i*r| (ties to the even code,
 * saturating at 6).
 * This is the activation quantiser that feeds each NVFP4 GEMM: page
 * "CURRENT_BUG.md - DeepSeek-V4 Blackwell NVFP4" (revision dd7af0c, section
 * "Root Cause Investigation") tests it on its own as one step of the MoE
 * path, and page "Current Bug: vLLM produces empty/garbage output" (revision
 * a51edd2, section "What the quant method does") shows why the direction of
 * its global scale must be fixed (a stored inverse read as a multiplier gave
 * NaN); here the direction is pinned and out-of-range blocks saturate.
 * Errors: EINVAL for null pointers or an unknown dtype; ESHAPE unless
 * rows >= 0, cols % 16 == 0, ld_x >= cols; EALIGN for misaligned pointers or
 * row pitch.  rows == 0 or cols == 0 is a no-op.
 */
int32_t nvfp4_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                       int64_t ld_x, const float* gs, uint8_t* codes, uint8_t* scales,
                       uint16_t* dq, void* stream);

/*
 * nvfp4_global_scale - per-slice global scales from the amax of each slice:
 * gs[b] = fp32(amax(x[b, 0:n]) / 2688), or 1.0 when the amax is 0
 * (2688 = 6 * 448 is the largest magnitude one block can encode).  Used for
 * weights (one scale per projection) and for warmup calibration of
 * activation scales.
 *   x        [batch, stride] of x_dtype, slice b = x[b, 0:n]; 16-byte aligned,
 *            stride*elem_size a multiple of 16, n a multiple of 8.
 *   gs_out   out [batch] float32.
 *   ws       workspace of at least nvfp4_global_scale_workspace_size(batch, n)
 *            bytes (16-byte aligned; may be NULL if that size is 0).
 * The maximum is order-independent, so the result is exact and deterministic.
 * The pages compute activation global scales from a warmup pass (page
 * "Current Bug: vLLM produces empty/garbage output", revision e8b289e,
 * section "Phase 1: CuTeDSL Shared Expert Kernel", and the MoE runner "with
 * warmup gs" in the standalone-chain table of revision a51edd2) and keep one
 * activation scale per layer input (revision a51edd2, "What the quant method
 * does": the per-expert input scales are collapsed to their maximum); this
 * call is that reduction, run over a warmup batch, a weight, or (for
 * per-batch scales) the batch itself.
 */
size_t nvfp4_global_scale_workspace_size(int64_t batch, int64_t n);
int32_t nvfp4_global_scale(const void* x, int32_t x_dtype, int64_t batch, int64_t n,
                           int64_t stride, float* gs_out, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * nvfp4_global_scale_noalloc - nvfp4_global_scale without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * partial maxima go to scratch memory the library holds on each device, so
 * the call allocates nothing.  Same arguments (minus ws, ws_bytes), results
 * and errors as nvfp4_global_scale, plus:
 *   - ESHAPE when nvfp4_global_scale_workspace_size(batch, n) exceeds
 *     NVFP4_NOALLOC_SCRATCH_BYTES (256 KiB: e.g. up to 64 slices of any
 *     length, or 65535 slices of up to 16384 elements);
 *   - EHIP if the scratch of the current device cannot be looked up.
 * The scratch is per device and shared by every call on it: it is fully
 * rewritten before it is read, so a call never depends on an earlier one,
 * but calls that overlap in time on one device (several streams or host
 * threads) race on it and give unspecified results.  `stream` must belong
 * to the current device.
 */
#define NVFP4_NOALLOC_SCRATCH_BYTES 262144
int32_t nvfp4_global_scale_noalloc(const void* x, int32_t x_dtype, int64_t batch, int64_t n,
                                   int64_t stride, float* gs_out, void* stream);

/*
 * moe_route_permute - top-k routing and the group-by-expert permutation.
 *   logits            [T, E] float32 router logits.
 *   topk_ids          out [T, k] int32: slot 0 is the largest logit; equal
 *                     logits are ordered by expert id (lower first).
 *   topk_w            out [T, k] float32: softmax over the k selected logits,
 *                     w_j = e_j / sum with e_j = exp(l_j - l_0) (float32
 *                     exponential by Cody-Waite reduction and a degree-8
 *                     Taylor polynomial, 0 below -80) and the sum taken in
 *                     slot order.
 *   expert_offsets    out [E+1] int32: rows of expert e are
 *                     [expert_offsets[e], expert_offsets[e+1]).
 *   sorted_token_ids  out [T*k] int32: token of each permuted row; within an
 *                     expert rows follow the flat index t*k + j.
 *   inv_perm          out [T, k] int32: the permuted row holding (t, j).
 * Top-k and scatter are what the routed experts have and the shared expert
 * lacks (page "Current Bug: vLLM produces empty/garbage output", e8b289e,
 * section "Phase 1: CuTeDSL Shared Expert Kernel").
 * Errors: EINVAL for null pointers; ESHAPE unless T >= 0,
 * 1 <= E <= NVFP4_MAX_EXPERTS, 1 <= k <= min(E, NVFP4_MAX_TOPK),
 * T*k < 2^31.  T == 0 writes expert_offsets = 0 and nothing else.
 */
int32_t moe_route_permute(const float* logits, int64_t T, int32_t E, int32_t k,
                          int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                          int32_t* sorted_token_ids, int32_t* inv_perm, void* stream);

/*
 * moe_route_permute_shared - moe_route_permute with n_shared always-on
 * shared experts folded in as extra groups, so that one grouped GEMM per
 * projection covers the routed and the shared experts of a layer.  The page
 * "Current Bug: vLLM produces empty/garbage output" (e8b289e, section
 * "Phase 1: CuTeDSL Shared Expert Kernel") describes a shared expert as an
 * MoE of one expert without routing, run by the same grouped kernel; here it
 * is one more expert that every token visits with weight 1.
 *   Each token has kk = k + n_shared slots: slots 0 .. k-1 exactly as
 *   moe_route_permute (ids, softmax weights over the k selected logits);
 *   slot k + s holds expert id E + s with weight 1.0f.
 *   topk_ids, topk_w, inv_perm   out [T, kk].
 *   expert_offsets               out [E + n_shared + 1]: groups 0 .. E-1 are
 *                                the routed experts, group E + s the shared
 *                                expert s (T rows, tokens in order).
 *   sorted_token_ids             out [T*kk], expert-major, flat index t*kk + j
 *                                within a group.
 * moe_combine over kk slots then adds each shared expert's output with weight
 * 1 after the routed slots, in slot order.  n_shared = 0 is moe_route_permute.
 * Errors: those of moe_route_permute, and ESHAPE unless n_shared >= 0,
 * k + n_shared <= NVFP4_MAX_TOPK, E + n_shared <= NVFP4_MAX_EXPERTS,
 * T*kk < 2^31.
 */
int32_t moe_route_permute_shared(const float* logits, int64_t T, int32_t E, int32_t k, int32_t n_shared,
                                 int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                                 int32_t* sorted_token_ids, int32_t* inv_perm, void* stream);

/*
 * nvfp4_grouped_gemm - grouped GEMM of two NVFP4 operands.
 *   For every group g and every row m in [group_offsets[g], group_offsets[g+1]):
 *     out[m, n] = alpha(g, n) * sum_k A[m, k] * W[g, n, k]
 *   where A and W are the block-scaled values e2m1 * e4m3 (without global
 *   scales) and alpha(g, n) = fp32(a_gs * w_gs[g, s]) for the column segment
 *   s with n_seg[s] <= n < n_seg[s+1].  This is the epilogue factor
 *   activation-global-scale x weight-global-scale of page revision a51edd2
 *   ("What the quant method does"); the per-segment weight scales are the
 *   page's dual global scales for fused weights (gate+up, q_a+kv; e8b289e,
 *   "Phase 2: CuTeDSL Attention Kernel").  Products are exact and sums are
 *   float32 (matrix-core accumulation), so results agree with the exact
 *   contraction to float32 summation error, not bitwise.
 *   a_codes, a_scales  A storage, [a_rows, K/2] and [a_rows, K/16].
 *   a_gs               ONE float32.
 *   a_row_index        [M] int32 or NULL: logical row m reads stored row
 *                      a_row_index[m] (the gather by sorted_token_ids);
 *                      NULL means row m is stored row m (then a_rows >= M).
 *   a_dq               [a_rows, K] f16 (uint16 storage) or NULL: the same A
 *                      dequantised without its global scale, as the dq
 *                      output of nvfp4_quantize or silu_mul_requant writes
 *                      it.  It MUST agree with a_codes/a_scales: a kernel
 *                      reads whichever form suits it (the matrix-core tiles
 *                      of the tiled layout copy it straight into local
 *                      memory),
 *                      and both give the same products.  Ignored when
 *                      a_rows * K * 2 >= 2^32.
 *   w_codes, w_scales  [G, N, K/2], [G, N, K/16] when w_layout is
 *                      NVFP4_LAYOUT_ROWS; when it is NVFP4_LAYOUT_TILED,
 *                      w_codes is the buffer nvfp4_prepare_weights wrote for
 *                      the same G, N, K and w_scales is ignored (may be NULL).
 *                      Both layouts give results within the float32
 *                      summation bound of the exact contraction (groups
 *                      with many rows may run on a different kernel, so
 *                      the two are not bitwise equal).
 *   w_gs               [G, n_segs] float32.
 *   n_seg              HOST array of n_segs+1 int32: 0 = n_seg[0] < ... <
 *                      n_seg[n_segs] = N.
 *   group_offsets      [G+1] int32, non-decreasing, 0 .. M.
 *   out                [M, ld_out] of out_dtype (F32 or BF16, rounded to
 *                      nearest-even), columns [0, N) written; rows outside
 *                      every group are left untouched.
 *   workspace          device memory of ws_bytes (16-byte aligned) or NULL:
 *                      see nvfp4_grouped_gemm_workspace_size.  Caller-owned;
 *                      calls that share one workspace must not overlap.
 * Errors: EINVAL for null pointers, an unknown dtype or layout; ESHAPE
 * unless 1 <= G <= NVFP4_MAX_EXPERTS, 1 <= n_segs <= NVFP4_MAX_SEGMENTS,
 * M >= 0, N >= 1, K >= 32 with K % 32 == 0 (K % 256 == 0 and K <= 2^24
 * for the tiled layout), ld_out >= N, a_rows >= 1 when M > 0 (and >= M when a_row_index
 * is NULL), n_seg increasing from 0 to N; EALIGN unless codes (and the tiled
 * buffer), a_dq and out are 16-byte aligned and scales 4-byte aligned.
 */
int32_t nvfp4_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                           int64_t a_rows, const int32_t* a_row_index, const uint16_t* a_dq,
                           const uint8_t* w_codes, const uint8_t* w_scales, int32_t w_layout,
                           const float* w_gs,
                           const int32_t* n_seg, int32_t n_segs,
                           const int32_t* group_offsets, int32_t G,
                           int64_t M, int64_t N, int64_t K,
                           void* out, int32_t out_dtype, int64_t ld_out,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * nvfp4_grouped_gemm_workspace_size - bytes of device workspace with which
 * nvfp4_grouped_gemm of these sizes and weight layout splits K (0: it never
 * does).  With few workgroups for the chip (tiled layout: few groups and
 * rows, up to 16 ranges; or one group whose 128-row tiles number at most 256
 * and whose A comes in f16 form, up to 8 ranges), K
 * is cut into ranges whose raw float32 partial sums are written to the
 * workspace and then added in range order by a second kernel
 * (deterministic), which applies alpha once.  A NULL or smaller workspace
 * runs the GEMM in one pass; results differ only by float32 summation order
 * (both within the documented bound).  Pure host function.
 */
size_t nvfp4_grouped_gemm_workspace_size(int32_t G, int64_t M, int64_t N, int64_t K, int32_t w_layout);

/*
 * nvfp4_grouped_gemm_silu_requant - the first grouped GEMM of the expert MLP
 * with SiLU(gate) * up and its NVFP4 re-quantisation in the epilogue: the
 * stacked gate_up projection (page e8b289e, "Phase 1": grouped GEMM, SiLU,
 * re-quant) without the float32 [M, 2I] intermediate.
 *   Equivalent to nvfp4_grouped_gemm(a_*, w_tiled, NVFP4_LAYOUT_TILED, w_gs,
 *   n_seg = {0, I, 2I}, group_offsets, G, M, N = 2I, K, out f32 [M, 2I])
 *   followed by silu_mul_requant(out, F32, M, I, 2I, h_gs, h_codes,
 *   h_scales, h_dq): every value of gate and up is formed as that GEMM
 *   writes it and goes through the same float32 steps, so codes, scales
 *   and h_dq are identical to the pair of calls.
 *   a_codes ... a_dq   as for nvfp4_grouped_gemm.
 *   w_tiled            the nvfp4_prepare_weights buffer of the stacked
 *                      [G, 2I, K] weights (gate rows [0, I), up rows
 *                      [I, 2I)); w_gs [G, 2] (gate, up).
 *   h_gs               ONE float32, the global scale of h.
 *   h_codes, h_scales  out [M, I/2], [M, I/16]; h_dq out [M, I] f16 or NULL
 *                      (as silu_mul_requant writes them).  Rows outside every
 *                      group are left untouched.
 *   workspace          device memory of ws_bytes (16-byte aligned) or NULL,
 *                      sized by nvfp4_grouped_gemm_workspace_size(G, M, 2I,
 *                      K, NVFP4_LAYOUT_TILED).  With it K is split exactly as
 *                      in nvfp4_grouped_gemm given the same workspace, and a
 *                      second kernel adds the partial sums in range order,
 *                      applies alpha and re-quantises SiLU(gate) * up, so the
 *                      equivalence above holds with that workspace passed to
 *                      both.  Caller-owned; calls that share one workspace
 *                      must not overlap.
 * Errors: EINVAL for null pointers; ESHAPE unless 1 <= G <=
 * NVFP4_MAX_EXPERTS, M >= 0, I >= 32 with I % 32 == 0, 256 <= K <= 2^24
 * with K % 256 == 0, a_rows as for nvfp4_grouped_gemm; EALIGN unless codes,
 * w_tiled, a_dq, h_codes and h_dq are 16-byte aligned and scales and global
 * scales 4-byte aligned.
 */
int32_t nvfp4_grouped_gemm_silu_requant(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                                        int64_t a_rows, const int32_t* a_row_index, const uint16_t* a_dq,
                                        const uint8_t* w_tiled, const float* w_gs,
                                        const int32_t* group_offsets, int32_t G, int64_t M, int64_t I,
                                        int64_t K, const float* h_gs, uint8_t* h_codes, uint8_t* h_scales,
                                        uint16_t* h_dq, void* workspace, size_t ws_bytes, void* stream);

/*
 * nvfp4_grouped_gemm_silu_f32 - the first grouped GEMM of the expert MLP with
 * h = SiLU(gate) * up written in float32, and the maxima of |h| that give its
 * global scale: the per-batch (dynamic) activation scale of the intermediate
 * without the float32 [M, 2I] gate_up.  The pages trace their failure to
 * activation global scales that did not match the data (page "Current Bug:
 * vLLM produces empty/garbage output", revision a51edd2, section "What the
 * quant method does"); a scale taken from the batch itself cannot be stale.
 *   Arguments a_codes ... K as for nvfp4_grouped_gemm_silu_requant.
 *   h              out [M, I] float32 (row pitch I, 16-byte aligned): every
 *                  value as silu_mul_requant forms it from the gate_up that
 *                  nvfp4_grouped_gemm writes (no split-K).  Rows outside
 *                  every group are left untouched.
 *   amax_partials  out [n_partials] float32, n_partials >=
 *                  nvfp4_grouped_gemm_silu_f32_partials(G, M, I): zeroed by
 *                  the call, then partial maxima of |h| (of rows inside the
 *                  groups); their maximum is max |h|.
 * Then nvfp4_global_scale(amax_partials as one slice of n_partials) gives
 * the same gs_h as silu_mul_global_scale of that gate_up, and
 * nvfp4_quantize(h, gs_h) the same codes, scales and f16 copy as
 * silu_mul_requant (both take the maximum, which does not depend on order,
 * and the same float32 steps).
 * Errors: as nvfp4_grouped_gemm_silu_requant; ESHAPE if n_partials is too
 * small; EALIGN unless h is 16-byte and amax_partials 4-byte aligned.
 */
size_t nvfp4_grouped_gemm_silu_f32_partials(int32_t G, int64_t M, int64_t I);
int32_t nvfp4_grouped_gemm_silu_f32(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                                    int64_t a_rows, const int32_t* a_row_index, const uint16_t* a_dq,
                                    const uint8_t* w_tiled, const float* w_gs,
                                    const int32_t* group_offsets, int32_t G, int64_t M, int64_t I,
                                    int64_t K, float* h, float* amax_partials, int64_t n_partials,
                                    void* stream);

/*
 * nvfp4_moe_expert_mlp - the routed experts' MLP in ONE persistent launch:
 * the first grouped GEMM over the stacked gate_up weights with SiLU(gate) *
 * up re-quantised in its epilogue, then the second grouped GEMM over the
 * down weights, taken from one device tile queue so that the second GEMM's
 * weight stream starts while the first GEMM's last tiles still run.  This is
 * the single persistent launch of a MegaMoE-style layer (page
 * "CURRENT_BUG.md - DeepSeek-V4 Blackwell NVFP4", section "Architecture
 * Notes", which describes a persistent grouped GEMM for MegaMoE) for the
 * pipeline of page "Current Bug: vLLM produces empty/garbage output"
 * (revision e8b289e, section "Phase 1: CuTeDSL Shared Expert Kernel": GEMM,
 * SiLU, re-quant, GEMM).
 *   Equivalent to nvfp4_grouped_gemm_silu_requant(x_codes, x_scales, x_gs,
 *   x_rows, sorted_token_ids, NULL, w1_tiled, w1_gs, expert_offsets, G, R,
 *   I, H, h_gs, h_codes, h_scales, NULL) followed by
 *   nvfp4_grouped_gemm(h_codes, h_scales, h_gs, R, NULL, NULL, w2_tiled,
 *   NULL, NVFP4_LAYOUT_TILED, w2_gs, {0, H}, 1, expert_offsets, G, R, H, I,
 *   y, NVFP4_DTYPE_BF16, H, NULL, 0): h is identical; y is identical where
 *   that second call streams its weights in 32-row slots (few rows per
 *   group, the decode regime) and within the float32 summation bound of the
 *   exact contraction in every case.  Every group is processed in 32-row
 *   slots, so the launch suits few rows per group; with many rows per group
 *   the two calls (matrix-core tiles) are faster.
 *   x_codes, x_scales  NVFP4 layer input [x_rows, H/2], [x_rows, H/16];
 *                      x_gs ONE float32.
 *   sorted_token_ids   [R] int32 or NULL: row m of the experts' input is
 *                      x row sorted_token_ids[m] (moe_route_permute).
 *   expert_offsets     [G+1] int32 (moe_route_permute / _shared).
 *   w1_tiled, w1_gs    nvfp4_prepare_weights buffer of the stacked [G, 2I, H]
 *                      weights (gate rows [0, I), up rows [I, 2I)) and
 *                      their [G, 2] global scales (gate, up).
 *   w2_tiled, w2_gs    nvfp4_prepare_weights buffer of [G, H, I] and [G, 1].
 *   h_gs               ONE float32, the global scale of h.
 *   h_codes, h_scales  out [R, I/2], [R, I/16] (also the second GEMM's A).
 *   y                  out [R, H] bf16 (uint16 storage).
 *   workspace          nvfp4_moe_expert_mlp_workspace_size(G, R) bytes of
 *                      device memory (4-byte aligned): the tile queue, a
 *                      status word and one completion counter per 32-row
 *                      slot, reset by the call itself.  Calls sharing a
 *                      workspace must not overlap.
 * Dependency waits are bounded (about 2^22 polls, or NVFP4MOE_SPIN_LIMIT
 * from the environment): if one gives up, the launch still finishes,
 * int32 workspace word 1 is set non-zero and the results are unspecified
 * (under NVFP4MOE_SYNC_CHECK=1 the call then returns NVFP4_EHIP).
 * Errors: EINVAL for null pointers; ESHAPE unless 1 <= G <=
 * NVFP4_MAX_EXPERTS, R >= 0, H and I are multiples of 256 in [256, 2^24], x_rows
 * as for nvfp4_grouped_gemm, the workspace is large enough; EALIGN as
 * stated.  R == 0 is a no-op.
 */
size_t nvfp4_moe_expert_mlp_workspace_size(int32_t G, int64_t R);
int32_t nvfp4_moe_expert_mlp(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                             int64_t x_rows, const int32_t* sorted_token_ids,
                             const int32_t* expert_offsets, int32_t G, int64_t R,
                             const uint8_t* w1_tiled, const float* w1_gs, const uint8_t* w2_tiled,
                             const float* w2_gs, int64_t H, int64_t I, const float* h_gs,
                             uint8_t* h_codes, uint8_t* h_scales, uint16_t* y, void* workspace,
                             size_t ws_bytes, void* stream);

/*
 * nvfp4_grouped_gemm_reads_dq - 1 if nvfp4_grouped_gemm with these sizes
 * (G groups, M rows, depth K, a_rows stored A rows) and weight layout reads
 * a_dq when it is given, else 0: the tiled layout's matrix-core tiles read
 * it, which run from 32 rows per group on average (16 where K <= 4096) and
 * for one group of at most 128 rows split over K.  Lets a caller produce the
 * f16 form of A only where it is used.  Pure host function; it
 * neither fails nor sets the last error.
 */
int32_t nvfp4_grouped_gemm_reads_dq(int32_t G, int64_t M, int64_t K, int64_t a_rows, int32_t w_layout);

/*
 * nvfp4_prepare_weights - rearrange NVFP4 weights [G, N, K] (row-major codes
 * and scales) into the tiled layout (NVFP4_LAYOUT_TILED) that
 * nvfp4_grouped_gemm streams with whole-cache-line loads.  It is a pure byte
 * permutation (plus zero padding of the last 16-row block): the GEMM's
 * results do not change.  Done once when weights are loaded; the row-major
 * buffers may be freed afterwards.
 *   w_codes [G, N, K/2], w_scales [G, N, K/16] (16-byte aligned).
 *   out     nvfp4_prepared_weight_bytes(G, N, K) bytes, 16-byte aligned.
 * Layout: rows in blocks of 32 (last block zero-padded), k in steps of 256,
 * each step two half-steps h of 128; tile (g, block, step) holds 4608
 * contiguous bytes, tiles ordered by g, block, step.  With lane
 * l = c + 32 kh (c = row in block, kh = 0, 1): bytes
 * [2048h + 1024i + 16l, +16) are code bytes [64h + 32kh + 16i, +16) of that
 * row's 128 code bytes of the step (i = 0, 1), and bytes
 * [4096 + 256h + 4l, +4) its scale bytes [8h + 4kh, +4) of the step's 16.
 * Errors: EINVAL for null pointers; ESHAPE unless G >= 1, N >= 1,
 * K % 256 == 0 and 256 <= K <= 2^24; EALIGN for misaligned pointers.
 */
size_t nvfp4_prepared_weight_bytes(int64_t G, int64_t N, int64_t K);
int32_t nvfp4_prepare_weights(const uint8_t* w_codes, const uint8_t* w_scales, int64_t G, int64_t N,
                              int64_t K, uint8_t* out, void* stream);

/*
 * silu_mul_requant - h = SiLU(gate) * up, re-quantised to NVFP4.
 *   gate_up  [M, ld] of in_dtype (F32 or BF16): gate in columns [0, I), up in
 *            [I, 2I) (the stacked gate_up order).
 *   gs_h     ONE float32, the global scale of h.
 *   h_codes  out [M, I/2]; h_scales out [M, I/16].
 *   h_dq     out [M, I] f16 or NULL: h dequantised without gs_h, as the dq
 *            output of nvfp4_quantize.
 * Per element in float32, each step one IEEE operation: e = exp(-g) (the
 * same exponential as moe_route_permute, +Inf above 88), s = g / (1 + e),
 * h = s * u; then the quantisation of nvfp4_quantize with gs_h.
 * This is the "SiLU -> re-quant" step between the two GEMMs of the expert
 * MLP on page "Current Bug: vLLM produces empty/garbage output" (revision
 * e8b289e, section "Phase 1: CuTeDSL Shared Expert Kernel"), applied to the
 * stacked gate_up output; the page keeps SiLU in BF16, here it stays float32
 * up to the re-quantisation (no intermediate rounding).
 * Errors: EINVAL for null pointers or an unknown dtype; ESHAPE unless M >= 0,
 * I % 16 == 0, ld >= 2I; EALIGN unless gate_up is 16-byte aligned and
 * ld*elem_size is a multiple of 16.
 */
int32_t silu_mul_requant(const void* gate_up, int32_t in_dtype, int64_t M, int64_t I,
                         int64_t ld, const float* gs_h, uint8_t* h_codes, uint8_t* h_scales,
                         uint16_t* h_dq, void* stream);

/*
 * silu_mul_global_scale - gs_out = fp32(amax(SiLU(gate)*up) / 2688) (1.0 if
 * the amax is 0), with h computed exactly as in silu_mul_requant: the warmup
 * calibration of the intermediate's global scale.
 *   ws  workspace of silu_mul_global_scale_workspace_size(M, I) bytes.
 */
size_t silu_mul_global_scale_workspace_size(int64_t M, int64_t I);
int32_t silu_mul_global_scale(const void* gate_up, int32_t in_dtype, int64_t M, int64_t I,
                              int64_t ld, float* gs_out, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * moe_combine - weighted sum of each token's k expert outputs, plus an
 * optional residual, back in token order.
 *   y         [T*k, H] of y_dtype (F32 or BF16), permuted rows.
 *   inv_perm  [T, k] int32, topk_w [T, k] float32 (from moe_route_permute).
 *   residual  [T, H] bf16 (uint16 storage, 16-byte aligned) or NULL.
 *   out       [T, H] bf16 (uint16 storage).
 * out[t] = bf16(acc) with acc = w_0*y[inv[t,0]], then acc = acc + w_j*y[inv[t,j]]
 * for j = 1..k-1, then (with a residual) acc = acc + residual[t], each product
 * and sum a separate float32 operation, one rounding to bf16 (nearest-even)
 * at the end.  This is the final scatter of the routed experts' outputs back
 * to the tokens, which the page keeps in BF16 (page "Current Bug: vLLM
 * produces empty/garbage output", revision e8b289e, section "Phase 3: Clean
 * up"); the residual lets a caller add the layer's skip connection (or a
 * separately computed shared expert) in the same pass without a second
 * bf16 rounding.
 * Errors: EINVAL for null pointers or an unknown dtype; ESHAPE unless T >= 0,
 * 1 <= k <= NVFP4_MAX_TOPK, H % 8 == 0; EALIGN unless y, residual and out are
 * 16-byte aligned.
 */
int32_t moe_combine(const void* y, int32_t y_dtype, const int32_t* inv_perm,
                    const float* topk_w, int64_t T, int32_t k, int64_t H, const uint16_t* residual,
                    uint16_t* out, void* stream);

/*
 * fp8_quantize_weight - block-scaled FP8 (E4M3) weights for the attention
 * output projection wo_a, which the pages run as an FP8 weight-only einsum
 * without an input scale (page e8b289e, "Phase 2: CuTeDSL Attention Kernel";
 * "CURRENT_BUG.md - DeepSeek-V4 Blackwell NVFP4", "Architecture Notes").
 *   w       [N, ld_w] float32 (16-byte aligned, ld_w % 4 == 0), columns [0, K).
 *   codes   out [N, K] E4M3 (FN) codes.
 *   scales  out [ceil(N/128), K/128] float32: one dequantisation scale per
 *           128 x 128 block, s = amax / 448 (1.0 for an all-zero block).
 * Per weight: q = w / s (float32 division), code = sign bit of w plus the
 * E4M3 magnitude nearest to |q| (ties to even, saturating at 448, never NaN).
 * Errors: EINVAL for null pointers; ESHAPE unless N >= 0, K >= 128 with
 * K % 128 == 0, ld_w >= K; EALIGN as stated.
 */
int32_t fp8_quantize_weight(const float* w, int64_t N, int64_t K, int64_t ld_w, uint8_t* codes,
                            float* scales, void* stream);

/*
 * fp8_weight_gemm - out = x . value(W)^T with bf16 activations x [M, ld_x]
 * (uint16 storage, columns [0, K)) and the FP8 weights of
 * fp8_quantize_weight: value(n, k) = e4m3(codes[n, k]) * scales[n/128, k/128].
 *   Every bf16 x E4M3 product is exact (bf16 matrix-core products); each
 *   128-wide k-block is summed in float32 and added to the result as
 *   result += scale * block_sum, in k order, so the result agrees with the
 *   exact sum to float32 summation error, not bitwise.
 *   out  [M, ld_out] of out_dtype (F32 or BF16, rounded to nearest-even).
 * Errors: EINVAL for null pointers or an unknown dtype; ESHAPE unless
 * M >= 0, N >= 1, K >= 128 with K % 128 == 0, ld_x >= K, ld_out >= N;
 * EALIGN unless x, its row pitch and the codes are 16-byte aligned.
 */
int32_t fp8_weight_gemm(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint8_t* w_codes,
                        const float* w_scales, int64_t N, void* out, int32_t out_dtype, int64_t ld_out,
                        void* stream);

/*
 * Measurement probes (not part of the pipeline).  The bench reports the
 * pipeline's rates against the vendor peaks and, as second denominators,
 * against what these simplest kernels reach on the same chip; the pages
 * publish no throughput of their own to compare with.
 *
 * nvfp4_probe_hbm_read - read `bytes` of device memory once with 16-byte
 * non-temporal loads, grid-stride over 2048 workgroups of 256 lanes, eight
 * loads in flight per lane.  Nothing is written unless the folded value of
 * the data equals one fixed 32-bit constant; `sink` is 4 bytes of device
 * memory for that case.  Errors: ESHAPE unless bytes >= 0 and
 * bytes % 16 == 0; EINVAL for null pointers; EALIGN unless buf is 16-byte
 * aligned.
 *
 * nvfp4_probe_mfma_f16 - `workgroups` workgroups of four waves; each wave
 * runs `iters` rounds of eight independent v_mfma_f32_32x32x16_f16 chains
 * on register operands that alternate between two sets of pseudo-random
 * values.  Floating-point operations: workgroups * 4 * iters * 8 * 32768.
 * `sink` as above (4 bytes, written only for one fixed float value).
 * Errors: ESHAPE unless iters >= 0 and 0 <= workgroups <= 65535; EINVAL for
 * a null sink.
 */
int32_t nvfp4_probe_hbm_read(const void* buf, int64_t bytes, void* sink, void* stream);
int32_t nvfp4_probe_mfma_f16(int64_t iters, int64_t workgroups, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4MOE_H */
