// Internal interface between the C ABI (capi.hip) and the gfx950 kernels
// (finalize_kernels.hip).  Not installed; the public interface is
// include/moe_finalize.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mf {

// What the kernel does after the FP32 routed sum.
enum class Epilogue : int {
    kRound,              // out = bf16(acc)
    kRmsNorm,            // out = bf16(acc * inv_rms(acc) * g),  g = w + gain_center
    kRmsNormWeightFirst, // z = acc * g; out = bf16(z * inv_rms(z))
    kBeam,               // out = bf16(bf16(acc) * routed_scale)
    kBeamNorm,           // s = as kBeam; out = bf16(s * inv_rms(s) * post_weight)
};

// Arguments of one launch; validated by the caller.
struct FinalizeArgs {
    const uint16_t *rows;     // BF16 row matrix (index map) or [cap, K, H] (token major)
    int64_t row_stride;       // elements between rows (index map only)
    int64_t num_rows;         // valid index range [0, num_rows) (index map only)
    const int32_t *idx;       // [T, K] index map, or nullptr for token major
    const void *weights;      // [T, K] FP32 or BF16
    bool weights_bf16;
    const uint16_t *gain;     // BF16 [H]: norm_weight / post_weight (nullable for kBeamNorm)
    uint16_t *out;            // BF16 [T, H]
    int32_t num_tokens;
    int32_t hidden;
    int32_t top_k;
    float eps;
    float gain_center;
    float routed_scale;
};

// Enqueue the finalize on `stream`; returns the launch status.
hipError_t launch_finalize(const FinalizeArgs &a, Epilogue epi, hipStream_t stream);

}  // namespace mf
