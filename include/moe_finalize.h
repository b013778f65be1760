/*
 * moe_finalize.h - C ABI of the MI355X (gfx950) MoE expert-output finalize
 * library (libmoe_finalize.so).
 *
 * The MoE finalize step turns the raw, unweighted rows that the second expert
 * GEMM wrote (one row per (token, expert slot)) into one hidden vector per
 * token: it gathers each token's top-k rows, sums them weighted by the routing
 * weights in FP32, optionally normalises the sum with a per-token RMSNorm and
 * writes BF16.  Sources (web pages, cited by title and section):
 *
 *   [TPF]  FlashInfer "flashinfer.comm.tp_moe_finalize_rmsnorm":
 *          description paragraph and Parameters list.
 *   [BEAM] vLLM "vllm.models.beam.nvidia.moe_finalize": beam_moe_finalize
 *          (docstring, Parameters and the argument checks of its wrapper).
 *   [RMOE] FlashInfer "flashinfer.fused_moe.trtllm_fp8_per_tensor_scale_routed_moe":
 *          Returns section (the producer's unfinalized triple).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Data pointers are DEVICE pointers owned by the caller; the library keeps
 *    no reference after the call returns and allocates nothing.  BF16 data is
 *    2 bytes per element (IEEE binary32 upper half).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    and the call returns without waiting.  No synchronisation with other
 *    streams is inserted; order producers and consumers on other streams
 *    with events [TPF description].
 *  - Arguments are validated on the host before any HIP call.  On a
 *    validation error nothing is launched and the output is untouched.
 *  - A call with zero output rows validates its arguments, launches nothing
 *    and returns MF_OK.
 *  - Every token count the entry points accept (up to INT32_MAX) is served:
 *    the pages set no limit on the number of tokens [TPF Parameters: output
 *    (num_tokens, 4096)].  A call whose grid would span more than 2^31
 *    work-items (one workgroup of up to 1024 threads per token, or one
 *    64-thread wave per four tokens at hidden 256 and top-k 1, per two at
 *    top-k 2-7 and at hidden 512 and top-k 1) runs as
 *    several launches on `stream`, in token order; the split is invisible
 *    to the caller.
 *  - The output must not overlap any input.  Calls on different streams may
 *    run concurrently when their outputs do not overlap.
 *  - Numerics: the routed sum is a chain of FP32 fused multiply-adds over
 *    the slots in ascending order starting from +0; FP32 -> BF16 conversion
 *    rounds to nearest, ties to even.  Normalised outputs are within one
 *    BF16 unit in the last place of the exactly rounded result; outputs
 *    without a norm are exact.
 *  - The library is stateless and needs no initialisation call.
 */
#ifndef MOE_FINALIZE_H
#define MOE_FINALIZE_H

#include <stdint.h>

/* Exported from the shared library even when it is built with hidden
 * default visibility. */
#if defined(__GNUC__) || defined(__clang__)
#define MF_API __attribute__((visibility("default")))
#else
#define MF_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum mf_status {
    MF_OK = 0,
    MF_ERR_NULL_POINTER = 1,   /* a required pointer is NULL                   */
    MF_ERR_BAD_SHAPE = 2,      /* a size is negative, inconsistent or outside
                                  the entry point's envelope                   */
    MF_ERR_BAD_DTYPE = 3,      /* weights_dtype is not MF_DTYPE_BF16/FP32      */
    MF_ERR_MISALIGNED = 4,     /* a pointer or row stride breaks the 16-byte
                                  alignment rule                               */
    MF_ERR_BAD_ARGUMENT = 5,   /* inconsistent optional arguments              */
    MF_ERR_LAUNCH_FAILED = 6   /* the HIP launch reported an error; see
                                  mf_last_error_message()                      */
};

/* Element type of expert_weights on the index-map entry points. */
enum mf_dtype {
    MF_DTYPE_BF16 = 1,
    MF_DTYPE_FP32 = 2
};

/*
 * moe_finalize_rmsnorm - index-map finalize fused with per-token RMSNorm
 * [TPF description and Parameters].
 *
 * For token t < num_tokens and slot k < top_k, i = expanded_idx_to_permuted_idx
 * [t*top_k + k] names row i of gemm2_permuted; an index outside [0, num_rows)
 * contributes nothing (no row is read for it, its weight is not used, and the
 * other weights are not rescaled).  With acc the FP32 weighted sum of the valid rows' first
 * `hidden` columns and g[h] = float(norm_weight[h]) + gain_center (FP32 add):
 *   weight_before_norm == 0:  out = acc / sqrt(mean(acc^2) + eps) * g
 *   weight_before_norm != 0:  z = acc * g;  out = z / sqrt(mean(z^2) + eps)
 * with the mean over the `hidden` elements of the token.
 *
 *   gemm2_permuted  BF16 [num_rows, row_stride]; rows in physical expert
 *                   order; only columns [0, hidden) are read.  Row starts
 *                   16-byte aligned: pointer 16-byte aligned and row_stride
 *                   (elements) a multiple of 8 and >= hidden.
 *   expert_weights  [num_tokens, top_k], contiguous, BF16 or FP32 as given by
 *                   weights_dtype; 16-byte aligned.
 *   expanded_idx_to_permuted_idx  int32 [num_tokens, top_k], contiguous,
 *                   16-byte aligned.
 *   norm_weight     BF16 [hidden], 16-byte aligned.
 *   output          BF16 [num_tokens, hidden], contiguous, 16-byte aligned.
 *   hidden, top_k   256 <= hidden <= 8192 with hidden % 256 == 0 and
 *                   1 <= top_k <= 32.  The page specialises to 4096 and 8;
 *                   the library accepts the token-major path's envelope
 *                   [BEAM] for the index map too.
 *   eps             added to the mean square inside the square root.
 *
 * Errors: NULL pointer when num_tokens > 0 (gemm2_permuted may be NULL when
 * num_rows == 0: every index is then invalid) -> MF_ERR_NULL_POINTER;
 * hidden or top_k outside the envelope, num_tokens < 0 or > INT32_MAX, num_rows < 0,
 * row_stride < hidden, or a row matrix (num_rows x row_stride) too large to
 * address -> MF_ERR_BAD_SHAPE; bad weights_dtype
 * -> MF_ERR_BAD_DTYPE; misaligned pointer or row_stride % 8 != 0 ->
 * MF_ERR_MISALIGNED.
 */
MF_API int moe_finalize_rmsnorm(const void *gemm2_permuted, int64_t num_rows,
                         int64_t row_stride, const void *expert_weights,
                         int32_t weights_dtype,
                         const int32_t *expanded_idx_to_permuted_idx,
                         const void *norm_weight, void *output,
                         int64_t num_tokens, int32_t hidden, int32_t top_k,
                         float eps, float gain_center,
                         int32_t weight_before_norm, void *stream);

/*
 * moe_finalize - index-map finalize without a norm: out = bf16(acc), the
 * finalized tensor that the producer returns when it finalizes itself in
 * place of the unfinalized (gemm2 output, weights, index map) triple [RMOE
 * Returns], with the gather, masking and FP32 reduction of [TPF description].
 *
 * Arguments and layout as moe_finalize_rmsnorm without the norm arguments.
 * Envelope: 256 <= hidden <= 8192 with hidden % 256 == 0, 1 <= top_k <= 32.
 * Errors as moe_finalize_rmsnorm.
 */
MF_API int moe_finalize(const void *gemm2_permuted, int64_t num_rows,
                 int64_t row_stride, const void *expert_weights,
                 int32_t weights_dtype,
                 const int32_t *expanded_idx_to_permuted_idx, void *output,
                 int64_t num_tokens, int32_t hidden, int32_t top_k,
                 void *stream);

/*
 * beam_moe_finalize - token-major finalize with BF16 rounding points and an
 * optional RMSNorm [BEAM beam_moe_finalize].
 *
 * Slot k of token t is the contiguous row expert_outputs[t, k, :]; there is no
 * index map and no masking.  For t < live_tokens:
 *   r = bf16(acc)                       acc = FP32 weighted sum over slots
 *   s = bf16(float(r) * routed_scale)   (FP32 product)
 *   has_norm == 0:  out = s
 *   has_norm != 0:  out = bf16(s / sqrt(mean(s^2) + post_eps) * pw)
 * where pw = float(post_weight[h]), or 1 when post_weight is NULL.  Rows and
 * weights of tokens >= live_tokens are never read.
 *
 *   expert_outputs  BF16 [capacity, top_k, hidden], contiguous, 16-byte aligned.
 *   expert_weights  FP32 [weight_rows, top_k], contiguous, 4-byte aligned,
 *                   weight_rows >= live_tokens.
 *   output          BF16 [live_tokens, hidden], contiguous, 16-byte aligned.
 *   post_weight     BF16 [hidden] or NULL; 16-byte aligned.
 *   Envelope: 1 <= top_k <= 32; 256 <= hidden <= 8192, hidden % 256 == 0;
 *   0 <= live_tokens <= capacity, live_tokens <= INT32_MAX.
 *
 * Errors: NULL expert_outputs/expert_weights/output (when live_tokens > 0)
 * -> MF_ERR_NULL_POINTER; envelope or size violations -> MF_ERR_BAD_SHAPE;
 * post_weight given with has_norm == 0 -> MF_ERR_BAD_ARGUMENT; misalignment
 * -> MF_ERR_MISALIGNED.
 */
MF_API int beam_moe_finalize(const void *expert_outputs, int64_t capacity,
                      int32_t top_k, int32_t hidden,
                      const float *expert_weights, int64_t weight_rows,
                      void *output, int64_t live_tokens,
                      const void *post_weight, float routed_scale,
                      float post_eps, int32_t has_norm, void *stream);

/*
 * mf_rmsnorm - standalone per-token RMSNorm of BF16 rows: the second step of
 * the unfused strategy (finalize first, normalise separately) that the
 * [BEAM] fused finalize pages keep for validation and benchmarking, with the
 * norm of [TPF] (eps inside the root, g = float(norm_weight) + gain_center
 * in FP32, weight before or after the statistics).  With x = float(input):
 *   weight_before_norm == 0:  out = x / sqrt(mean(x^2) + eps) * g
 *   weight_before_norm != 0:  z = x * g;  out = z / sqrt(mean(z^2) + eps)
 * moe_finalize followed by mf_rmsnorm is the unfused counterpart of
 * moe_finalize_rmsnorm (it rounds the sum to BF16 in between).
 *
 *   input        BF16 [num_tokens, row_stride], row_stride % 8 == 0 and
 *                >= hidden; only columns [0, hidden) are read.
 *   norm_weight  BF16 [hidden];  output  BF16 [num_tokens, hidden], contiguous.
 *   All 16-byte aligned; hidden in the envelope of moe_finalize.
 * Errors as moe_finalize_rmsnorm.
 */
MF_API int mf_rmsnorm(const void *input, int64_t row_stride, const void *norm_weight,
                      void *output, int64_t num_tokens, int32_t hidden, float eps,
                      float gain_center, int32_t weight_before_norm, void *stream);

/*
 * beam_moe_finalize_norm_residual_norm - token-major finalize fused with the
 * residual add and the next layer's norm [BEAM
 * beam_moe_finalize_norm_residual_norm].  The page defines the operation as
 * equal to its unfused strategy: beam_moe_finalize (with its optional
 * post-norm) followed by a residual/next-norm consumer whose body is not on
 * the page.  This library reads that consumer as (PARITY UNPINNED against the
 * pages for the scales and the rounding point of hidden):
 *   y          = beam_moe_finalize output of token t (BF16)
 *   hidden     = bf16(scale_x * y + scale_res * residual[t])
 *   normalized = bf16(hidden / sqrt(mean(hidden^2) + next_eps) * nw)
 * where nw = next_weight (or 1 when NULL) and normalized is computed from
 * hidden as stored.  The page passes its `scales` pair as (scale_x,
 * scale_res), or (1, 1) when the pair is absent.
 *
 *   expert_outputs, expert_weights, capacity, top_k, hidden, routed_scale,
 *   post_weight, post_eps, has_post_norm   as beam_moe_finalize
 *   residual        BF16 [num_tokens, hidden], contiguous, 16-byte aligned
 *   next_weight     BF16 [hidden] or NULL (only with has_next_norm)
 *   hidden_out      BF16 [num_tokens, hidden], contiguous
 *   normalized_out  BF16 [num_tokens, hidden], required iff has_next_norm
 *   num_tokens      tokens to finalize: <= capacity and <= weight_rows
 * Errors as beam_moe_finalize; a norm weight without its norm ->
 * MF_ERR_BAD_ARGUMENT.
 */
MF_API int beam_moe_finalize_norm_residual_norm(
    const void *expert_outputs, int64_t capacity, int32_t top_k, int32_t hidden,
    const float *expert_weights, int64_t weight_rows, const void *residual,
    const void *post_weight, const void *next_weight, void *hidden_out,
    void *normalized_out, int64_t num_tokens, float routed_scale, float post_eps,
    float next_eps, float scale_x, float scale_res, int32_t has_post_norm,
    int32_t has_next_norm, void *stream);

/*
 * beam_norm_residual_norm - the consumer of the unfused strategy on its own
 * (second step of the [BEAM] unfused baseline): optional post-norm of the
 * BF16 rows x (as in beam_moe_finalize, rounded to BF16), then hidden and
 * normalized as in beam_moe_finalize_norm_residual_norm.  Same reading,
 * PARITY UNPINNED against the pages.
 *
 *   x         BF16 [num_tokens, row_stride], row_stride % 8 == 0, >= hidden
 *   other arguments as beam_moe_finalize_norm_residual_norm.
 */
MF_API int beam_norm_residual_norm(const void *x, int64_t row_stride, const void *residual,
                                   const void *post_weight, const void *next_weight,
                                   void *hidden_out, void *normalized_out,
                                   int64_t num_tokens, int32_t hidden, float post_eps,
                                   float next_eps, float scale_x, float scale_res,
                                   int32_t has_post_norm, int32_t has_next_norm,
                                   void *stream);

/* Static, human-readable name of a status code (never NULL). */
MF_API const char *mf_status_string(int status);

/* Message of the last MF_ERR_LAUNCH_FAILED on the calling thread ("" if none). */
MF_API const char *mf_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FINALIZE_H */
