/*
 * CPU oracle for the MoE expert-output finalize path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the GPU library is checked against.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path never calls it and shares no code, header or table with it.
 *
 * Sources (web pages; cited by title and section):
 *   [TPF]  FlashInfer API page "flashinfer.comm.tp_moe_finalize_rmsnorm":
 *          description paragraph and the Parameters list.
 *   [BEAM] vLLM API page "vllm.models.beam.nvidia.moe_finalize":
 *          function beam_moe_finalize (docstring, Parameters, wrapper body).
 *   [RMOE] FlashInfer API page
 *          "flashinfer.fused_moe.trtllm_fp8_per_tensor_scale_routed_moe":
 *          Returns section (the unfinalized triple when do_finalize is off).
 *   [BEAM] also: beam_moe_finalize_norm_residual_norm (docstring and wrapper)
 *          and, through its unfused strategy, the consumer it calls after
 *          beam_moe_finalize, beam_norm_residual_norm, whose body is not on
 *          the page.  oracle_beam_norm_residual_norm below is the plainest
 *          reading of that consumer (see there); PARITY UNPINNED against
 *          the pages for the two scales and the rounding point of hidden.
 *   The unfused strategy of beam_moe_finalize_norm_residual_norm on [BEAM]
 *   (finalize first, normalise in a separate step, kept for validation and
 *   benchmarking) motivates oracle_rmsnorm: the [TPF] norm applied to rows
 *   that were already rounded to BF16.
 *
 * Precision policy.  Where the pages fix a precision it is kept exactly:
 *   - the routed reduction is FP32 (weights of either dtype become FP32 and
 *     the sum stays FP32) [TPF description];
 *   - gain_center is added to norm_weight in FP32 [TPF Parameters, gain_center];
 *   - the token-major path rounds to BF16 after the reduction and again after
 *     routed_scale [BEAM docstring, routed_scale].
 * Everything the pages leave open (the RMS statistics, the normalisation and
 * the affine multiply) is computed in binary64 and rounded to BF16 once.
 *
 * Readings of points the pages leave open (each is pinned by a test):
 *   - the reduction runs over slots k = 0..K-1 in ascending order, as one
 *     fused multiply-add per slot, starting from +0;
 *   - an index i contributes only if 0 <= i < num_rows; an invalid slot is
 *     skipped entirely (its row and weight are not touched, so NaN there
 *     cannot leak) and the remaining weights are not renormalised;
 *   - RMSNorm is per token over the hidden dimension with divisor H and
 *     y = z / sqrt(mean(z^2) + eps);
 *   - with weight_before_norm the effective weight multiplies the FP32 sum
 *     before the statistics and is not applied again afterwards;
 *   - routed_scale multiplies the BF16-rounded sum in FP32 (one FP32
 *     rounding), and the product is rounded to BF16;
 *   - FP32/FP64 -> BF16 is round-to-nearest, ties to even; NaN becomes a
 *     quiet NaN with the input's sign.
 *
 * Parity pins (tests/test_oracle_*.py): library routines (torch CPU float ->
 * bfloat16, torch rms_norm in float64), exact rational arithmetic on tiny
 * shapes, closed forms, invariants and error bounds.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

/* ---------------------------------------------------------------- BF16 ---- */

/* A BF16 value is the upper half of a binary32 pattern, so widening is exact. */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * Round a binary64 value to the nearest BF16 (8 significant bits, binary32
 * exponent range), ties to even, with a single rounding.  Binary32 inputs are
 * passed widened, which is exact.
 */
uint16_t oracle_round_to_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);

    int e;
    (void)frexp(a, &e);              /* a = m * 2^e with 0.5 <= m < 1        */
    int ulp_exp = e - 8;             /* 8 significant bits                    */
    if (ulp_exp < -133)              /* below 2^-126 the grid is 2^-133       */
        ulp_exp = -133;
    double q = ldexp(a, -ulp_exp);   /* exact: a in units of the last place  */
    double lo = floor(q);
    double rem = q - lo;             /* exact                                 */
    double r = lo;
    if (rem > 0.5 || (rem == 0.5 && fmod(lo, 2.0) != 0.0))
        r = lo + 1.0;
    double v = ldexp(r, ulp_exp);    /* exact: at most 9 significant bits     */
    if (v >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u);

    float f = (float)v;              /* exact: v lies on the BF16 grid        */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFFu));
}

/* ------------------------------------------------------ routed reduction -- */

/*
 * FP32 routed sum for one token of the index-map layout [TPF description].
 *   rows      BF16 matrix, row r starts at rows + r*row_stride (elements)
 *   idx       the token's K entries of expanded_idx_to_permuted_idx
 *   w_f32/w_bf16  the token's K routing weights (exactly one is non-NULL)
 *   acc       out: H binary32 sums
 */
static void routed_sum_index_map(const uint16_t *rows, int64_t num_rows,
                                 int64_t row_stride, const int32_t *idx,
                                 const float *w_f32, const uint16_t *w_bf16,
                                 int32_t hidden, int32_t top_k, float *acc)
{
    for (int32_t h = 0; h < hidden; ++h)
        acc[h] = 0.0f;
    for (int32_t k = 0; k < top_k; ++k) {
        int64_t i = idx[k];
        if (i < 0 || i >= num_rows)
            continue;                            /* contributes nothing */
        float w = w_f32 ? w_f32[k] : oracle_bf16_to_f32(w_bf16[k]);
        const uint16_t *row = rows + i * row_stride;
        for (int32_t h = 0; h < hidden; ++h)
            acc[h] = fmaf(w, oracle_bf16_to_f32(row[h]), acc[h]);
    }
}

/* FP32 routed sum for one token of the token-major layout [BEAM docstring]:
 * slot k of this token is the contiguous row expert_outputs[t, k, :]. */
static void routed_sum_token_major(const uint16_t *token_rows, const float *w,
                                   int32_t hidden, int32_t top_k, float *acc)
{
    for (int32_t h = 0; h < hidden; ++h)
        acc[h] = 0.0f;
    for (int32_t k = 0; k < top_k; ++k) {
        const uint16_t *row = token_rows + (int64_t)k * hidden;
        for (int32_t h = 0; h < hidden; ++h)
            acc[h] = fmaf(w[k], oracle_bf16_to_f32(row[h]), acc[h]);
    }
}

/* ------------------------------------------------------------ RMSNorm ----- */

/* 1 / sqrt(mean(z^2) + eps) over H values, in binary64. */
static double inv_rms(const double *z, int32_t hidden, double eps)
{
    double ss = 0.0;
    for (int32_t h = 0; h < hidden; ++h)
        ss += z[h] * z[h];
    return 1.0 / sqrt(ss / (double)hidden + eps);
}

/* --------------------------------------------------------- entry points -- */

/*
 * The routed reduction alone for every token: acc_out[t, h] (binary32).
 * weights_is_fp32 selects the dtype of `weights` (FP32 or BF16) [TPF
 * Parameters, expert_weights].
 */
int oracle_routed_sum(const uint16_t *gemm2_permuted, int64_t num_rows,
                      int64_t row_stride, const void *weights,
                      int32_t weights_is_fp32, const int32_t *idx,
                      float *acc_out, int64_t num_tokens, int32_t hidden,
                      int32_t top_k)
{
    if (hidden <= 0 || top_k <= 0 || num_tokens < 0 || row_stride < hidden)
        return -1;
    for (int64_t t = 0; t < num_tokens; ++t) {
        const float *wf = weights_is_fp32 ? (const float *)weights + t * top_k : NULL;
        const uint16_t *wb = weights_is_fp32 ? NULL : (const uint16_t *)weights + t * top_k;
        routed_sum_index_map(gemm2_permuted, num_rows, row_stride,
                             idx + t * top_k, wf, wb, hidden, top_k,
                             acc_out + t * hidden);
    }
    return 0;
}

/* Finalize without a norm: out = bf16(routed FP32 sum).  This is what the
 * producer's do_finalize step returns in place of the unfinalized triple
 * [RMOE Returns], computed by the index-map rule of [TPF description]. */
int oracle_moe_finalize(const uint16_t *gemm2_permuted, int64_t num_rows,
                        int64_t row_stride, const void *weights,
                        int32_t weights_is_fp32, const int32_t *idx,
                        uint16_t *output, int64_t num_tokens, int32_t hidden,
                        int32_t top_k)
{
    if (hidden <= 0 || top_k <= 0 || num_tokens < 0 || row_stride < hidden)
        return -1;
    float *acc = (float *)malloc(sizeof(float) * (size_t)hidden);
    if (!acc)
        return -2;
    for (int64_t t = 0; t < num_tokens; ++t) {
        const float *wf = weights_is_fp32 ? (const float *)weights + t * top_k : NULL;
        const uint16_t *wb = weights_is_fp32 ? NULL : (const uint16_t *)weights + t * top_k;
        routed_sum_index_map(gemm2_permuted, num_rows, row_stride,
                             idx + t * top_k, wf, wb, hidden, top_k, acc);
        for (int32_t h = 0; h < hidden; ++h)
            output[t * hidden + h] = oracle_round_to_bf16((double)acc[h]);
    }
    free(acc);
    return 0;
}

/*
 * Finalize fused with per-token RMSNorm [TPF description and Parameters]:
 *   g  = f32(norm_weight) + gain_center              (FP32 add)
 *   z  = weight_before_norm ? acc * g : acc
 *   y  = z / sqrt(mean(z^2) + eps) * (weight_before_norm ? 1 : g)
 */
int oracle_moe_finalize_rmsnorm(const uint16_t *gemm2_permuted, int64_t num_rows,
                                int64_t row_stride, const void *weights,
                                int32_t weights_is_fp32, const int32_t *idx,
                                const uint16_t *norm_weight, uint16_t *output,
                                int64_t num_tokens, int32_t hidden, int32_t top_k,
                                float eps, float gain_center,
                                int32_t weight_before_norm)
{
    if (hidden <= 0 || top_k <= 0 || num_tokens < 0 || row_stride < hidden)
        return -1;
    float *acc = (float *)malloc(sizeof(float) * (size_t)hidden);
    float *g = (float *)malloc(sizeof(float) * (size_t)hidden);
    double *z = (double *)malloc(sizeof(double) * (size_t)hidden);
    if (!acc || !g || !z) {
        free(acc); free(g); free(z);
        return -2;
    }
    for (int32_t h = 0; h < hidden; ++h)
        g[h] = oracle_bf16_to_f32(norm_weight[h]) + gain_center;
    for (int64_t t = 0; t < num_tokens; ++t) {
        const float *wf = weights_is_fp32 ? (const float *)weights + t * top_k : NULL;
        const uint16_t *wb = weights_is_fp32 ? NULL : (const uint16_t *)weights + t * top_k;
        routed_sum_index_map(gemm2_permuted, num_rows, row_stride,
                             idx + t * top_k, wf, wb, hidden, top_k, acc);
        for (int32_t h = 0; h < hidden; ++h)
            z[h] = weight_before_norm ? (double)acc[h] * (double)g[h] : (double)acc[h];
        double inv = inv_rms(z, hidden, (double)eps);
        for (int32_t h = 0; h < hidden; ++h) {
            double y = z[h] * inv;
            if (!weight_before_norm)
                y *= (double)g[h];
            output[t * hidden + h] = oracle_round_to_bf16(y);
        }
    }
    free(acc); free(g); free(z);
    return 0;
}

/*
 * Standalone RMSNorm of BF16 rows (the second step of the unfused strategy):
 * the [TPF] norm with x = f32(input) in place of the FP32 routed sum.
 *   input   BF16 rows, row t starts at input + t*row_stride (elements)
 */
int oracle_rmsnorm(const uint16_t *input, int64_t row_stride,
                   const uint16_t *norm_weight, uint16_t *output,
                   int64_t num_tokens, int32_t hidden, float eps,
                   float gain_center, int32_t weight_before_norm)
{
    if (hidden <= 0 || num_tokens < 0 || row_stride < hidden)
        return -1;
    float *g = (float *)malloc(sizeof(float) * (size_t)hidden);
    double *z = (double *)malloc(sizeof(double) * (size_t)hidden);
    if (!g || !z) {
        free(g); free(z);
        return -2;
    }
    for (int32_t h = 0; h < hidden; ++h)
        g[h] = oracle_bf16_to_f32(norm_weight[h]) + gain_center;
    for (int64_t t = 0; t < num_tokens; ++t) {
        const uint16_t *x = input + t * row_stride;
        for (int32_t h = 0; h < hidden; ++h) {
            double v = (double)oracle_bf16_to_f32(x[h]);
            z[h] = weight_before_norm ? v * (double)g[h] : v;
        }
        double inv = inv_rms(z, hidden, (double)eps);
        for (int32_t h = 0; h < hidden; ++h) {
            double y = z[h] * inv;
            if (!weight_before_norm)
                y *= (double)g[h];
            output[t * hidden + h] = oracle_round_to_bf16(y);
        }
    }
    free(g); free(z);
    return 0;
}

/*
 * Token-major finalize [BEAM beam_moe_finalize]: for each of the first
 * live_tokens tokens,
 *   r = bf16(acc);  s = bf16(f32(r) * routed_scale)   (FP32 product)
 *   out = s                                            without a norm
 *   out = bf16(s / sqrt(mean(s^2) + post_eps) * pw)    with a norm
 * where pw is post_weight (or 1 when post_weight is NULL).  Rows of tokens
 * at or beyond live_tokens are never read.
 */
int oracle_beam_moe_finalize(const uint16_t *expert_outputs, int64_t capacity,
                             int32_t top_k, int32_t hidden,
                             const float *expert_weights, uint16_t *output,
                             int64_t live_tokens, const uint16_t *post_weight,
                             float routed_scale, float post_eps, int32_t has_norm)
{
    if (hidden <= 0 || top_k <= 0 || live_tokens < 0 || live_tokens > capacity)
        return -1;
    float *acc = (float *)malloc(sizeof(float) * (size_t)hidden);
    double *s = (double *)malloc(sizeof(double) * (size_t)hidden);
    uint16_t *sb = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)hidden);
    if (!acc || !s || !sb) {
        free(acc); free(s); free(sb);
        return -2;
    }
    for (int64_t t = 0; t < live_tokens; ++t) {
        routed_sum_token_major(expert_outputs + t * top_k * (int64_t)hidden,
                               expert_weights + t * top_k, hidden, top_k, acc);
        for (int32_t h = 0; h < hidden; ++h) {
            uint16_t r = oracle_round_to_bf16((double)acc[h]);
            float scaled = oracle_bf16_to_f32(r) * routed_scale;
            sb[h] = oracle_round_to_bf16((double)scaled);
            s[h] = (double)oracle_bf16_to_f32(sb[h]);
        }
        uint16_t *out = output + t * (int64_t)hidden;
        if (!has_norm) {
            memcpy(out, sb, sizeof(uint16_t) * (size_t)hidden);
            continue;
        }
        double inv = inv_rms(s, hidden, (double)post_eps);
        for (int32_t h = 0; h < hidden; ++h) {
            double y = s[h] * inv;
            if (post_weight)
                y *= (double)oracle_bf16_to_f32(post_weight[h]);
            out[h] = oracle_round_to_bf16(y);
        }
    }
    free(acc); free(s); free(sb);
    return 0;
}

/*
 * Post-norm, residual add and next norm of BF16 rows x: the consumer that
 * the unfused strategy of [BEAM] beam_moe_finalize_norm_residual_norm calls
 * after beam_moe_finalize.  Its definition is not on the pages; the reading
 * taken here (PARITY UNPINNED against the pages):
 *   y      = has_post ? bf16(x / sqrt(mean(x^2) + post_eps) * pw) : x
 *            (pw = post_weight, or 1 when NULL; the norm of beam_moe_finalize)
 *   hidden = bf16(scale_x * y + scale_res * residual)
 *            (the wrapper passes the scales pair, or (1, 1) when it is None,
 *            so they are read as multipliers of the two summands)
 *   normalized = bf16(hidden / sqrt(mean(hidden^2) + next_eps) * nw)
 *            (nw = next_weight or 1; computed from hidden as stored in BF16,
 *            only when has_next)
 *   x, residual  BF16 rows; row t of x at x + t*row_stride, of residual at
 *                residual + t*hidden.
 */
int oracle_beam_norm_residual_norm(const uint16_t *x, int64_t row_stride,
                                   const uint16_t *residual,
                                   const uint16_t *post_weight,
                                   const uint16_t *next_weight,
                                   uint16_t *hidden_out, uint16_t *normalized_out,
                                   int64_t num_tokens, int32_t hidden,
                                   float post_eps, float next_eps,
                                   float scale_x, float scale_res,
                                   int32_t has_post, int32_t has_next)
{
    if (hidden <= 0 || num_tokens < 0 || row_stride < hidden)
        return -1;
    double *v = (double *)malloc(sizeof(double) * (size_t)hidden);
    if (!v)
        return -2;
    for (int64_t t = 0; t < num_tokens; ++t) {
        const uint16_t *xr = x + t * row_stride;
        const uint16_t *rr = residual + t * (int64_t)hidden;
        uint16_t *hr = hidden_out + t * (int64_t)hidden;
        for (int32_t h = 0; h < hidden; ++h)
            v[h] = (double)oracle_bf16_to_f32(xr[h]);
        if (has_post) {
            double inv = inv_rms(v, hidden, (double)post_eps);
            for (int32_t h = 0; h < hidden; ++h) {
                double y = v[h] * inv;
                if (post_weight)
                    y *= (double)oracle_bf16_to_f32(post_weight[h]);
                v[h] = (double)oracle_bf16_to_f32(oracle_round_to_bf16(y));
            }
        }
        for (int32_t h = 0; h < hidden; ++h) {
            double sum = (double)scale_x * v[h] +
                         (double)scale_res * (double)oracle_bf16_to_f32(rr[h]);
            hr[h] = oracle_round_to_bf16(sum);
            v[h] = (double)oracle_bf16_to_f32(hr[h]);
        }
        if (!has_next)
            continue;
        double inv = inv_rms(v, hidden, (double)next_eps);
        uint16_t *nr = normalized_out + t * (int64_t)hidden;
        for (int32_t h = 0; h < hidden; ++h) {
            double y = v[h] * inv;
            if (next_weight)
                y *= (double)oracle_bf16_to_f32(next_weight[h]);
            nr[h] = oracle_round_to_bf16(y);
        }
    }
    free(v);
    return 0;
}

/*
 * [BEAM] beam_moe_finalize_norm_residual_norm: beam_moe_finalize of the
 * first num_tokens tokens (with its optional post-norm) followed by
 * oracle_beam_norm_residual_norm without a second post-norm, exactly the
 * page's unfused strategy.  weight rows >= num_tokens, capacity >= num_tokens.
 */
int oracle_beam_moe_finalize_norm_residual_norm(
    const uint16_t *expert_outputs, int64_t capacity, int32_t top_k,
    int32_t hidden, const float *expert_weights, const uint16_t *residual,
    const uint16_t *post_weight, const uint16_t *next_weight,
    uint16_t *hidden_out, uint16_t *normalized_out, int64_t num_tokens,
    float routed_scale, float post_eps, float next_eps, float scale_x,
    float scale_res, int32_t has_post, int32_t has_next)
{
    if (num_tokens < 0 || num_tokens > capacity)
        return -1;
    uint16_t *fin = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(num_tokens > 0 ? num_tokens : 1) *
                                       (size_t)hidden);
    if (!fin)
        return -2;
    int rc = oracle_beam_moe_finalize(expert_outputs, capacity, top_k, hidden,
                                      expert_weights, fin, num_tokens, post_weight,
                                      routed_scale, post_eps, has_post);
    if (rc == 0)
        rc = oracle_beam_norm_residual_norm(fin, hidden, residual, NULL, next_weight,
                                            hidden_out, normalized_out, num_tokens,
                                            hidden, 0.0f, next_eps, scale_x, scale_res,
                                            0, has_next);
    free(fin);
    return rc;
}
