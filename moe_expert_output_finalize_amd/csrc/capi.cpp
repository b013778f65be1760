// C ABI of libmoe_finalize.so: argument validation, then mf::launch_finalize.
//
// Plain C++ with no HIP types: every check runs on the host before any HIP
// call, so a rejected call has no side effect, and the tests can build this
// file with an ordinary host compiler under AddressSanitizer and
// UndefinedBehaviorSanitizer against a recording stand-in for the launcher.
// The checks are the C form of the parameter contracts on the FlashInfer
// page "flashinfer.comm.tp_moe_finalize_rmsnorm" (Parameters: shapes, dtypes,
// unit-stride rows with a row stride that is a multiple of 8 elements,
// 16-byte alignment) and of the argument checks in beam_moe_finalize on the
// vLLM page "vllm.models.beam.nvidia.moe_finalize" (1 <= top_k <= 32, hidden
// a multiple of 256 in [256, 8192], live rows <= capacity, weight rows >=
// live rows, post_weight only with a norm, nothing to do for zero live rows).
// The FlashInfer page specialises its finalize+RMSNorm to hidden 4096 and
// top-k 8; here every entry point accepts the wider envelope of the vLLM
// checks, 4096 / 8 included.
#include <stdint.h>
#include <stdio.h>

#include "args.hpp"
#include "moe_finalize.h"

namespace {

thread_local char g_last_error[256] = "";

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool hidden_in_envelope(int32_t hidden) { return hidden >= 256 && hidden <= 8192 && hidden % 256 == 0; }

int launch(const mf::FinalizeArgs &a, mf::Layout layout, mf::Epilogue epi, void *stream)
{
    const int err = mf::launch_finalize(a, layout, epi, stream);
    if (err != 0) {
        snprintf(g_last_error, sizeof g_last_error, "kernel launch failed: %s (%d)",
                 mf::launch_error_string(err), err);
        return MF_ERR_LAUNCH_FAILED;
    }
    g_last_error[0] = '\0';
    return MF_OK;
}

// Checks shared by the two index-map entry points.  Returns MF_OK and fills
// `a`, or an error status.
int check_index_map(const void *gemm2_permuted, int64_t num_rows, int64_t row_stride,
                    const void *expert_weights, int32_t weights_dtype, const int32_t *idx,
                    void *output, int64_t num_tokens, int32_t hidden, int32_t top_k,
                    mf::FinalizeArgs &a)
{
    if (num_tokens < 0 || num_tokens > INT32_MAX || num_rows < 0)
        return MF_ERR_BAD_SHAPE;
    // The row matrix must be addressable: row_stride * num_rows elements.
    if (row_stride < hidden || (num_rows > 0 && row_stride > INT64_MAX / 2 / num_rows))
        return MF_ERR_BAD_SHAPE;
    if (weights_dtype != MF_DTYPE_BF16 && weights_dtype != MF_DTYPE_FP32)
        return MF_ERR_BAD_DTYPE;
    if (row_stride % 8 != 0)
        return MF_ERR_MISALIGNED;
    if (num_tokens > 0) {
        if ((num_rows > 0 && !gemm2_permuted) || !expert_weights || !idx || !output)
            return MF_ERR_NULL_POINTER;
        if (!aligned(gemm2_permuted, 16) || !aligned(expert_weights, 16) || !aligned(idx, 16) ||
            !aligned(output, 16))
            return MF_ERR_MISALIGNED;
    }
    a = mf::FinalizeArgs{};
    a.rows = static_cast<const uint16_t *>(gemm2_permuted);
    a.row_stride = row_stride;
    a.num_rows = num_rows;
    a.idx = idx;
    a.weights = expert_weights;
    a.weights_bf16 = weights_dtype == MF_DTYPE_BF16;
    a.out = static_cast<uint16_t *>(output);
    a.num_tokens = num_tokens;
    a.hidden = hidden;
    a.top_k = top_k;
    return MF_OK;
}

}  // namespace

extern "C" {

int moe_finalize_rmsnorm(const void *gemm2_permuted, int64_t num_rows, int64_t row_stride,
                         const void *expert_weights, int32_t weights_dtype,
                         const int32_t *expanded_idx_to_permuted_idx, const void *norm_weight,
                         void *output, int64_t num_tokens, int32_t hidden, int32_t top_k,
                         float eps, float gain_center, int32_t weight_before_norm, void *stream)
{
    if (!hidden_in_envelope(hidden) || top_k < 1 || top_k > 32)
        return MF_ERR_BAD_SHAPE;
    mf::FinalizeArgs a;
    const int rc = check_index_map(gemm2_permuted, num_rows, row_stride, expert_weights,
                                   weights_dtype, expanded_idx_to_permuted_idx, output,
                                   num_tokens, hidden, top_k, a);
    if (rc != MF_OK)
        return rc;
    if (num_tokens == 0)
        return MF_OK;
    if (!norm_weight)
        return MF_ERR_NULL_POINTER;
    if (!aligned(norm_weight, 16))
        return MF_ERR_MISALIGNED;
    a.gain = static_cast<const uint16_t *>(norm_weight);
    a.eps = eps;
    a.gain_center = gain_center;
    return launch(a, mf::Layout::kIndexMap,
                  weight_before_norm ? mf::Epilogue::kRmsNormWeightFirst : mf::Epilogue::kRmsNorm,
                  stream);
}

int moe_finalize(const void *gemm2_permuted, int64_t num_rows, int64_t row_stride,
                 const void *expert_weights, int32_t weights_dtype,
                 const int32_t *expanded_idx_to_permuted_idx, void *output, int64_t num_tokens,
                 int32_t hidden, int32_t top_k, void *stream)
{
    if (!hidden_in_envelope(hidden) || top_k < 1 || top_k > 32)
        return MF_ERR_BAD_SHAPE;
    mf::FinalizeArgs a;
    const int rc = check_index_map(gemm2_permuted, num_rows, row_stride, expert_weights,
                                   weights_dtype, expanded_idx_to_permuted_idx, output,
                                   num_tokens, hidden, top_k, a);
    if (rc != MF_OK)
        return rc;
    if (num_tokens == 0)
        return MF_OK;
    return launch(a, mf::Layout::kIndexMap, mf::Epilogue::kRound, stream);
}

int beam_moe_finalize(const void *expert_outputs, int64_t capacity, int32_t top_k, int32_t hidden,
                      const float *expert_weights, int64_t weight_rows, void *output,
                      int64_t live_tokens, const void *post_weight, float routed_scale,
                      float post_eps, int32_t has_norm, void *stream)
{
    if (top_k < 1 || top_k > 32 || !hidden_in_envelope(hidden))
        return MF_ERR_BAD_SHAPE;
    if (capacity < 0 || live_tokens < 0 || live_tokens > capacity || live_tokens > INT32_MAX ||
        weight_rows < live_tokens)
        return MF_ERR_BAD_SHAPE;
    if (post_weight && !has_norm)
        return MF_ERR_BAD_ARGUMENT;
    if (live_tokens == 0)
        return MF_OK;
    if (!expert_outputs || !expert_weights || !output)
        return MF_ERR_NULL_POINTER;
    if (!aligned(expert_outputs, 16) || !aligned(expert_weights, 4) || !aligned(output, 16) ||
        !aligned(post_weight, 16))
        return MF_ERR_MISALIGNED;
    mf::FinalizeArgs a{};
    a.rows = static_cast<const uint16_t *>(expert_outputs);
    a.row_stride = hidden;
    a.num_rows = capacity;   // unused: token-major slots are never masked
    a.idx = nullptr;
    a.weights = expert_weights;
    a.weights_bf16 = false;
    a.gain = static_cast<const uint16_t *>(post_weight);
    a.out = static_cast<uint16_t *>(output);
    a.num_tokens = live_tokens;
    a.hidden = hidden;
    a.top_k = top_k;
    a.eps = post_eps;
    a.routed_scale = routed_scale;
    return launch(a, mf::Layout::kTokenMajor,
                  has_norm ? mf::Epilogue::kBeamNorm : mf::Epilogue::kBeam, stream);
}

int mf_rmsnorm(const void *input, int64_t row_stride, const void *norm_weight, void *output,
               int64_t num_tokens, int32_t hidden, float eps, float gain_center,
               int32_t weight_before_norm, void *stream)
{
    if (!hidden_in_envelope(hidden) || num_tokens < 0 || num_tokens > INT32_MAX ||
        row_stride < hidden || (num_tokens > 0 && row_stride > INT64_MAX / 2 / num_tokens))
        return MF_ERR_BAD_SHAPE;
    if (row_stride % 8 != 0)
        return MF_ERR_MISALIGNED;
    if (num_tokens == 0)
        return MF_OK;
    if (!input || !norm_weight || !output)
        return MF_ERR_NULL_POINTER;
    if (!aligned(input, 16) || !aligned(norm_weight, 16) || !aligned(output, 16))
        return MF_ERR_MISALIGNED;
    mf::FinalizeArgs a{};
    a.rows = static_cast<const uint16_t *>(input);
    a.row_stride = row_stride;
    a.num_rows = num_tokens;
    a.gain = static_cast<const uint16_t *>(norm_weight);
    a.out = static_cast<uint16_t *>(output);
    a.num_tokens = num_tokens;
    a.hidden = hidden;
    a.top_k = 1;
    a.eps = eps;
    a.gain_center = gain_center;
    return launch(a, mf::Layout::kDirect,
                  weight_before_norm ? mf::Epilogue::kRmsNormWeightFirst : mf::Epilogue::kRmsNorm,
                  stream);
}

int beam_moe_finalize_norm_residual_norm(
    const void *expert_outputs, int64_t capacity, int32_t top_k, int32_t hidden,
    const float *expert_weights, int64_t weight_rows, const void *residual,
    const void *post_weight, const void *next_weight, void *hidden_out, void *normalized_out,
    int64_t num_tokens, float routed_scale, float post_eps, float next_eps, float scale_x,
    float scale_res, int32_t has_post_norm, int32_t has_next_norm, void *stream)
{
    if (top_k < 1 || top_k > 32 || !hidden_in_envelope(hidden))
        return MF_ERR_BAD_SHAPE;
    if (capacity < 0 || num_tokens < 0 || num_tokens > capacity || num_tokens > INT32_MAX ||
        weight_rows < num_tokens)
        return MF_ERR_BAD_SHAPE;
    if ((post_weight && !has_post_norm) || (next_weight && !has_next_norm))
        return MF_ERR_BAD_ARGUMENT;
    if (num_tokens == 0)
        return MF_OK;
    if (!expert_outputs || !expert_weights || !residual || !hidden_out ||
        (has_next_norm && !normalized_out))
        return MF_ERR_NULL_POINTER;
    if (!aligned(expert_outputs, 16) || !aligned(expert_weights, 4) || !aligned(residual, 16) ||
        !aligned(post_weight, 16) || !aligned(next_weight, 16) || !aligned(hidden_out, 16) ||
        !aligned(normalized_out, 16))
        return MF_ERR_MISALIGNED;
    mf::FinalizeArgs a{};
    a.rows = static_cast<const uint16_t *>(expert_outputs);
    a.row_stride = hidden;
    a.num_rows = capacity;   // unused: token-major slots are never masked
    a.weights = expert_weights;
    a.gain = static_cast<const uint16_t *>(post_weight);
    a.out = static_cast<uint16_t *>(hidden_out);
    a.num_tokens = num_tokens;
    a.hidden = hidden;
    a.top_k = top_k;
    a.eps = post_eps;
    a.routed_scale = routed_scale;
    a.residual = static_cast<const uint16_t *>(residual);
    a.gain2 = static_cast<const uint16_t *>(next_weight);
    a.out2 = static_cast<uint16_t *>(normalized_out);
    a.eps2 = next_eps;
    a.scale_x = scale_x;
    a.scale_res = scale_res;
    a.has_post = has_post_norm != 0;
    a.has_next = has_next_norm != 0;
    return launch(a, mf::Layout::kTokenMajor, mf::Epilogue::kResidualNorm, stream);
}

int beam_norm_residual_norm(const void *x, int64_t row_stride, const void *residual,
                            const void *post_weight, const void *next_weight, void *hidden_out,
                            void *normalized_out, int64_t num_tokens, int32_t hidden,
                            float post_eps, float next_eps, float scale_x, float scale_res,
                            int32_t has_post_norm, int32_t has_next_norm, void *stream)
{
    if (!hidden_in_envelope(hidden) || num_tokens < 0 || num_tokens > INT32_MAX ||
        row_stride < hidden || (num_tokens > 0 && row_stride > INT64_MAX / 2 / num_tokens))
        return MF_ERR_BAD_SHAPE;
    if (row_stride % 8 != 0)
        return MF_ERR_MISALIGNED;
    if ((post_weight && !has_post_norm) || (next_weight && !has_next_norm))
        return MF_ERR_BAD_ARGUMENT;
    if (num_tokens == 0)
        return MF_OK;
    if (!x || !residual || !hidden_out || (has_next_norm && !normalized_out))
        return MF_ERR_NULL_POINTER;
    if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(post_weight, 16) ||
        !aligned(next_weight, 16) || !aligned(hidden_out, 16) || !aligned(normalized_out, 16))
        return MF_ERR_MISALIGNED;
    mf::FinalizeArgs a{};
    a.rows = static_cast<const uint16_t *>(x);
    a.row_stride = row_stride;
    a.num_rows = num_tokens;
    a.gain = static_cast<const uint16_t *>(post_weight);
    a.out = static_cast<uint16_t *>(hidden_out);
    a.num_tokens = num_tokens;
    a.hidden = hidden;
    a.top_k = 1;
    a.eps = post_eps;
    a.routed_scale = 1.0f;   // bf16(bf16(x) * 1) == x: the rounding points are exact here
    a.residual = static_cast<const uint16_t *>(residual);
    a.gain2 = static_cast<const uint16_t *>(next_weight);
    a.out2 = static_cast<uint16_t *>(normalized_out);
    a.eps2 = next_eps;
    a.scale_x = scale_x;
    a.scale_res = scale_res;
    a.has_post = has_post_norm != 0;
    a.has_next = has_next_norm != 0;
    return launch(a, mf::Layout::kDirect, mf::Epilogue::kResidualNorm, stream);
}

const char *mf_status_string(int status)
{
    switch (status) {
    case MF_OK: return "ok";
    case MF_ERR_NULL_POINTER: return "a required pointer is NULL";
    case MF_ERR_BAD_SHAPE: return "a size is negative, inconsistent or outside the supported envelope";
    case MF_ERR_BAD_DTYPE: return "unsupported weights dtype";
    case MF_ERR_MISALIGNED: return "a pointer or row stride is not 16-byte aligned";
    case MF_ERR_BAD_ARGUMENT: return "inconsistent optional arguments (a norm weight without its norm)";
    case MF_ERR_LAUNCH_FAILED: return "the HIP kernel launch failed";
    default: return "unknown status";
    }
}

const char *mf_last_error_message(void) { return g_last_error; }

}  // extern "C"
