// Internal interface between the C ABI (capi.cpp) and the gfx950 kernels
// (finalize_kernels.hip).  Plain C++ with no HIP types, so that the C ABI's
// host code also builds with an ordinary host compiler (the sanitizer build
// of the tests links it against a recording stand-in for launch_finalize).
// Not installed; the public interface is include/moe_finalize.h.
#pragma once

#include <stdint.h>

namespace mf {

// Where a token's slot rows come from.
enum class Layout : int {
    kIndexMap,    // row idx[t, k] of a [num_rows, row_stride] matrix; invalid -> skipped
    kTokenMajor,  // row (t * K + k) of a [capacity * K, hidden] matrix
    kDirect,      // one slot, row t of a [T, row_stride] matrix, weight 1
};

// What the kernel does after the FP32 routed sum.
enum class Epilogue : int {
    kRound,              // out = bf16(acc)
    kRmsNorm,            // out = bf16(acc * inv_rms(acc) * g),  g = w + gain_center
    kRmsNormWeightFirst, // z = acc * g; out = bf16(z * inv_rms(z))
    kBeam,               // out = bf16(bf16(acc) * routed_scale)
    kBeamNorm,           // s = as kBeam; out = bf16(s * inv_rms(s) * post_weight)
    kResidualNorm,       // s = as kBeam; y = has_post ? bf16(s * inv_rms(s) * post_weight) : s;
                         // out = h = bf16(scale_x * y + scale_res * residual);
                         // out2 = bf16(h * inv_rms(h) * next_weight) when has_next
};

// Arguments of one call; validated by the caller.  Token t of the call
// reads and writes the rows of token t; a launch covers the tokens
// [token_base, token_base + gridDim.x).
struct FinalizeArgs {
    const uint16_t *rows;     // BF16 row matrix (see Layout)
    int64_t row_stride;       // elements between rows (index map, direct)
    int64_t num_rows;         // valid index range [0, num_rows) (index map only)
    const int32_t *idx;       // [T, K] index map, or nullptr for token major
    const void *weights;      // [T, K] FP32 or BF16
    bool weights_bf16;
    const uint16_t *gain;     // BF16 [H]: norm_weight / post_weight (nullable for kBeamNorm)
    uint16_t *out;            // BF16 [T, H]
    int64_t num_tokens;       // tokens of the whole call
    int64_t token_base;       // first token of this launch (set by the launcher)
    int32_t hidden;
    int32_t top_k;
    float eps;
    float gain_center;
    float routed_scale;
    // kResidualNorm only
    const uint16_t *residual; // BF16 [T, H]
    const uint16_t *gain2;    // BF16 [H] next_weight (nullable)
    uint16_t *out2;           // BF16 [T, H] normalized (when has_next)
    float eps2;               // next_eps
    float scale_x, scale_res;
    bool has_post, has_next;
};

// Enqueue the finalize of all num_tokens tokens on `stream` (a hipStream_t),
// in as many launches as the grid limit requires.  Returns 0 or the HIP error
// code of the first failed launch.  Supported pairs: index map with kRound /
// kRmsNorm / kRmsNormWeightFirst; token major with kBeam / kBeamNorm /
// kResidualNorm; direct with kRmsNorm / kRmsNormWeightFirst / kResidualNorm
// (routed_scale 1).
int launch_finalize(const FinalizeArgs &a, Layout layout, Epilogue epi, void *stream);

// Text of a code returned by launch_finalize (never NULL).
const char *launch_error_string(int code);

}  // namespace mf
