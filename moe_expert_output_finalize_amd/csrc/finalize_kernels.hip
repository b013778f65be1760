// gfx950 kernels for the MoE expert-output finalize.
//
// What is computed (sources are web pages, cited by title and section):
//  - FlashInfer "flashinfer.comm.tp_moe_finalize_rmsnorm", description and
//    Parameters: per token, gather the rows an index map selects (an index
//    outside [0, num_rows) contributes nothing), sum them weighted by the
//    routing weights in FP32, then RMSNorm with eps inside the root and an
//    effective weight norm_weight + gain_center (FP32), applied either to the
//    sum before the statistics or to the normalised value.
//  - vLLM "vllm.models.beam.nvidia.moe_finalize", beam_moe_finalize: the same
//    reduction over token-major rows [t, k, :], rounded to BF16, multiplied by
//    routed_scale and rounded to BF16 again before an optional RMSNorm.
//
// Mapping onto CDNA4.  The path moves ~70 KB per token and does ~1 FP32 op
// per byte, so it is bound by HBM bandwidth and uses no matrix cores:
//  - one workgroup per token; hidden/8 threads-or-fewer each own VPT 16-byte
//    column vectors of the token (vector j = lane + i * blockDim), so every
//    wave reads 1 KiB contiguous runs of each gathered row;
//  - the token's indices and weights are uniform, so they live in SGPRs (or
//    in VGPR lanes read back per slot) and validity is a scalar decision:
//    invalid slots issue no memory traffic;
//  - up to 16 row vectors per thread are in flight: all of a token's rows
//    when they fit (top-k 8 everywhere, top-k 16 at one vector per thread);
//    otherwise index-map slots stream through a rolling window (the rows of
//    slot s + W are issued once slot s is reduced) and token-major slots,
//    one contiguous block per token, arrive in batches;
//  - a call whose grid would exceed 2^31 work-items runs as several
//    launches, each finalizing the tokens from its token_base on;
//  - the FP32 sum, the sum of squares and the normalised values stay in
//    VGPRs; the cross-lane sum uses DPP row operations, the cross-wave sum
//    one LDS exchange and barrier;
//  - BF16 rounding is the CDNA4 packed convert (nearest even), two values
//    per instruction, and results leave as 16-byte buffer stores through a
//    resource spanning the output row, with device-scope cache policy;
//  - workgroup b takes token b: consecutive tokens run at the same time on
//    the eight XCDs (workgroups are dispatched to them in turn), so rows of
//    one expert that sit next to each other in memory are fetched together.
//    (Giving each XCD a contiguous token range instead measured 7% slower.)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "args.hpp"
#include "plan.hpp"

#ifndef MF_NONTEMPORAL_ROWS
#define MF_NONTEMPORAL_ROWS 1   // gathered rows are read exactly once
#endif
// Cache-policy operand of the output stores (CDNA4 buffer store: bit 0 sc0,
// bit 1 nt, bit 4 sc1).  Device-scope sc1 stores measured 1.5-2 % faster
// than non-temporal ones and 6 % faster than the default policy, with the
// gathered rows still read non-temporally.
#ifndef MF_STORE_POLICY
#define MF_STORE_POLICY 16
#endif
// Cache-policy operand of row loads through buffer resources (the streaming
// path): nt, as the global loads of the batch path.
#ifndef MF_ROW_LOAD_POLICY
#define MF_ROW_LOAD_POLICY 2
#endif

namespace mf {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// s_waitcnt operand on gfx9: vmcnt(0), expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;
// The kernel's own LDS: block_sum's two banks of per-wave partial sums.
constexpr int kStaticLds = 2 * kMaxWaves * sizeof(float);

// ------------------------------------------------------------ BF16 -------

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Element e (0..7) of a 16-byte vector of BF16 values, widened exactly.
__device__ __forceinline__ float elem(const u32x4 &v, int e)
{
    const uint32_t u = v[e >> 1];
    return (e & 1) ? bf16_hi(u) : bf16_lo(u);
}

// Round two FP32 values to BF16 (nearest, ties to even) and pack them, the
// first in the low half: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// sx * y + sr * r rounded once to BF16 (by pack_bf16x2), returned as the
// FP32 value to pack.  Each product of an FP32 scale and a BF16 value has at
// most 32 significant bits, so both are exact in binary64 and the fused
// multiply-add rounds their sum once; that binary64 sum is then rounded to
// FP32 to odd (an inexact result keeps its last bit set), which has 16 bits
// more than BF16, so the final round to nearest even sees no false tie and
// gives the BF16 rounding of the binary64 sum.  FP32 arithmetic instead
// (a multiply, a fused multiply-add, then BF16) rounds up to three times.
__device__ __forceinline__ float affine_to_odd(float sx, float y, float sr, float r)
{
    const double d = __builtin_fma((double)sx, (double)y, (double)sr * (double)r);
    const float f = (float)d;
    const uint32_t b = __float_as_uint(f);
    if ((double)f == d || f != f || (b & 1u))
        return f;
    // inexact and even: the neighbour on d's side (0 moves to the smallest
    // subnormal of its sign, infinity back to the largest finite value)
    return __uint_as_float(__builtin_fabs(d) > __builtin_fabs((double)f) ? b + 1u : b - 1u);
}

// ------------------------------------------------------------ memory -----

__device__ __forceinline__ u32x4 load_row_vec(const u32x4 *p)
{
#if MF_NONTEMPORAL_ROWS
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

// A row of hidden 512 (64 vectors) of zeros, never written: a lane of a
// multi-token wave reads it in place of a row it must not touch.
__device__ __align__(16) u32x4 zero_row[64];

// Buffer resource word 3 for raw (unformatted, unswizzled) access on gfx9.
constexpr int kRawBufferWord3 = 0x00020000;

// Resource spanning one output row of `bytes` bytes (uniform per workgroup).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_resource(uint16_t *row, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(row, 0, (int)bytes, kRawBufferWord3);
}

__device__ __forceinline__ void store_out_vec(__amdgpu_buffer_rsrc_t row, uint32_t byte_off,
                                              const u32x4 &v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, row, byte_off, 0, MF_STORE_POLICY);
}

// Vector j of a row of nv 16-byte vectors at p, or zeros for j >= nv: a
// buffer load bounded at the row's end, for teams with more threads than
// vectors.  A per-lane branch instead (load, else zero the registers) makes
// the compiler drain every load in flight before the zeroing, which
// serialised a token's gathers.
template <int POL>
__device__ __forceinline__ u32x4 load_vec_bounded(const void *p, int nv, int j)
{
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, nv * 16, kRawBufferWord3);
    return __builtin_amdgcn_raw_buffer_load_b128(r, j * 16, 0, POL);
}

template <bool BF16>
__device__ __forceinline__ float load_weight(const void *w, int64_t i)
{
    if constexpr (BF16)
        return __uint_as_float((uint32_t)static_cast<const uint16_t *>(w)[i] << 16);
    else
        return static_cast<const float *>(w)[i];
}

// ------------------------------------------------------------ reduction --

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Value of lane `l` (a constant) of v, as a wave-uniform scalar.
__device__ __forceinline__ int lane_value(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float lane_value(float v, int l)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Sum of v over the workgroup, returned to every thread.  All threads of the
// workgroup must call it (it contains a barrier when there are several waves).
// Two sums in one kernel use different banks, so the second's LDS writes
// cannot overtake a slower wave's reads of the first.  Within a wave the sum
// is the 16-lane DPP butterfly of each row (all 16 lanes end with the same
// bits), then the four rows in order.
__device__ __forceinline__ float block_sum(float v, int bank = 0)
{
    v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);   // row_half_mirror: 8-lane sums
    v += dpp_mov<0x140>(v);   // row_mirror: 16-lane sums
    const int iv = __builtin_bit_cast(int, v);
    float s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0)) +
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16)) +
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32)) +
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48));
    const int waves = blockDim.x / kWave;
    if (waves == 1)
        return s;
    __shared__ float part[2][kMaxWaves];
    if ((threadIdx.x & (kWave - 1)) == 0)
        part[bank][threadIdx.x / kWave] = s;
    __syncthreads();
    s = 0.0f;
    for (int i = 0; i < waves; ++i)
        s += part[bank][i];
    return s;
}

// Sum of the squares of acc over this lane's token's row.  One token per
// workgroup: each lane's FMA chain over its vectors, then block_sum.
// TPW > 1 tokens per wave (hidden 256 and 512): the order is that of one
// token per wave at these sizes, where lane l holds vector l: each vector's
// 8 squares by an FMA chain, each block of 16 vectors by the 16-lane DPP
// butterfly, then the blocks in order, ((B0 + B1) + B2) + B3.  A lane here
// holds vector l % LPT + LPT i of its token (LPT = 64 / TPW lanes per
// token): with 16 lanes, vector i is block i; with 32, block 2i in the
// token's first row of lanes and 2i + 1 in its second; with 8, half of
// block i / 2, whose halves the butterfly's last step adds.  So kernels of
// different layouts over the same rows, such as the fused residual path and
// its standalone consumer, compute the same sum bit for bit.
template <int VPT, int TPW>
__device__ __forceinline__ float row_sum_sq(const float (&acc)[VPT][8], int bank = 0)
{
    if constexpr (TPW == 1) {
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < VPT; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                ss = __builtin_fmaf(acc[i][e], acc[i][e], ss);   // idle vectors hold 0
        return block_sum(ss, bank);
    } else {
        float r[VPT];
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            float v = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v = __builtin_fmaf(acc[i][e], acc[i][e], v);
            v += dpp_mov<0xB1>(v);
            v += dpp_mov<0x4E>(v);
            v += dpp_mov<0x141>(v);
            if constexpr (TPW != 8)
                v += dpp_mov<0x140>(v);
            r[i] = v;
        }
        if constexpr (TPW == 8) {
            static_assert(VPT % 2 == 0, "two 8-vector halves per block");
            float s = r[0] + r[1];
#pragma unroll
            for (int b = 1; b < VPT / 2; ++b)
                s += r[2 * b] + r[2 * b + 1];
            return s;
        } else if constexpr (TPW == 4) {
            float s = r[0];
#pragma unroll
            for (int i = 1; i < VPT; ++i)
                s += r[i];
            return s;
        } else {
            static_assert(TPW == 2, "2, 4 or 8 tokens per wave");
            float lo = lane_value(r[0], 0) + lane_value(r[0], 16);
            float hi = lane_value(r[0], 32) + lane_value(r[0], 48);
#pragma unroll
            for (int i = 1; i < VPT; ++i) {
                lo = (lo + lane_value(r[i], 0)) + lane_value(r[i], 16);
                hi = (hi + lane_value(r[i], 32)) + lane_value(r[i], 48);
            }
            return (threadIdx.x & 32) ? hi : lo;
        }
    }
}


// ------------------------------------------------------------ kernel -----

// What follows a token's FP32 routed sum `acc`: the epilogue EPI and the
// stores of the workgroup's output row(s), which start at token t_row and
// span out_nv 16-byte vectors (one row, or TPW adjacent rows).  gv
// holds the norm weight (or post weight) vectors and rv the token's residual
// vectors, as the epilogue needs.  All threads of the workgroup call it (the
// norms contain a barrier).
template <Epilogue EPI, int VPT, bool EXACT, int TPW>
__device__ __forceinline__ void finish_token(float (&acc)[VPT][8], const u32x4 (&gv)[VPT],
                                             const u32x4 (&rv)[VPT], const FinalizeArgs &a,
                                             int64_t t_row, int out_nv, int lane, int team)
{
    constexpr bool kNorm = EPI == Epilogue::kRmsNorm || EPI == Epilogue::kRmsNormWeightFirst ||
                           EPI == Epilogue::kBeamNorm;
    constexpr bool kBeamRounding = EPI == Epilogue::kBeam || EPI == Epilogue::kBeamNorm ||
                                   EPI == Epilogue::kResidualNorm;
    const int nv = a.hidden >> 3;
    // Vector i of this lane: column col(i) of its token's row, position st(i)
    // among the workgroup's output vectors (TPW adjacent rows).
    auto col = [&](int i) {
        return TPW > 1 ? lane % (kWave / TPW) + (kWave / TPW) * i : lane + i * team;
    };
    auto st = [&](int i) { return TPW > 1 ? lane / (kWave / TPW) * nv + col(i) : col(i); };
    const __amdgpu_buffer_rsrc_t out_row =
        row_resource(a.out + t_row * (int64_t)a.hidden, (uint32_t)out_nv * 16u);
    // Lanes past the row (teams with more threads than vectors, the lanes of
    // tokens past the last) store outside the resource, which drops them.
    auto store = [&](int i, const u32x4 &o) { store_out_vec(out_row, (uint32_t)st(i) * 16u, o); };

    if constexpr (EPI == Epilogue::kRound) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                o[q] = pack_bf16x2(acc[i][2 * q], acc[i][2 * q + 1]);
            store(i, o);
        }
        return;
    }

    if constexpr (kBeamRounding) {
        // r = bf16(acc); s = bf16(r * routed_scale); s is kept widened in acc.
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t r = pack_bf16x2(acc[i][2 * q], acc[i][2 * q + 1]);
                const uint32_t s = pack_bf16x2(bf16_lo(r) * a.routed_scale,
                                               bf16_hi(r) * a.routed_scale);
                o[q] = s;
                acc[i][2 * q] = bf16_lo(s);
                acc[i][2 * q + 1] = bf16_hi(s);
            }
            if constexpr (EPI == Epilogue::kBeam)
                store(i, o);
        }
        if constexpr (EPI == Epilogue::kBeam)
            return;
    }

    if constexpr (EPI == Epilogue::kResidualNorm) {
        // Optional post-norm of s, rounded to BF16.
        if (a.has_post) {
            const float ss = row_sum_sq<VPT, TPW>(acc, 0);
            const float inv = rsqrtf(ss / (float)a.hidden + a.eps);
#pragma unroll
            for (int i = 0; i < VPT; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float y0 = acc[i][2 * q] * inv, y1 = acc[i][2 * q + 1] * inv;
                    if (a.gain) {
                        y0 *= elem(gv[i], 2 * q);
                        y1 *= elem(gv[i], 2 * q + 1);
                    }
                    const uint32_t p = pack_bf16x2(y0, y1);
                    acc[i][2 * q] = bf16_lo(p);
                    acc[i][2 * q + 1] = bf16_hi(p);
                }
        }
        // hidden = bf16(scale_x * y + scale_res * residual), one rounding,
        // kept widened in acc.  With scales of +-1 (the default pair (1, 1))
        // the FP32 sum of the two BF16 values is already that rounding: it
        // is exact unless their exponents differ by more than 16, and then
        // both it and the exact sum round to the larger value; other scales
        // take affine_to_odd.  The branch is uniform.
        auto add_residual = [&](auto sum) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                u32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t p = pack_bf16x2(sum(acc[i][2 * q], elem(rv[i], 2 * q)),
                                                   sum(acc[i][2 * q + 1], elem(rv[i], 2 * q + 1)));
                    o[q] = p;
                    acc[i][2 * q] = bf16_lo(p);
                    acc[i][2 * q + 1] = bf16_hi(p);
                }
                store(i, o);
            }
        };
        const bool unit_scales = (a.scale_x == 1.0f || a.scale_x == -1.0f) &&
                                 (a.scale_res == 1.0f || a.scale_res == -1.0f);
        if (unit_scales)
            add_residual([&](float y, float r) { return __builtin_fmaf(a.scale_x, y, a.scale_res * r); });
        else
            add_residual([&](float y, float r) { return affine_to_odd(a.scale_x, y, a.scale_res, r); });
        if (!a.has_next)
            return;
        // normalized = bf16(hidden * inv_rms(hidden) * next_weight)
        u32x4 nv2[VPT];
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int j = col(i);
            nv2[i] = (u32x4){0u, 0u, 0u, 0u};
            if (a.gain2)
                nv2[i] = EXACT ? reinterpret_cast<const u32x4 *>(a.gain2)[j]
                               : load_vec_bounded<0>(a.gain2, nv, j);
        }
        const float ss = row_sum_sq<VPT, TPW>(acc, 1);
        const float inv = rsqrtf(ss / (float)a.hidden + a.eps2);
        const __amdgpu_buffer_rsrc_t out2_row =
            row_resource(a.out2 + t_row * (int64_t)a.hidden, (uint32_t)out_nv * 16u);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float y0 = acc[i][2 * q] * inv, y1 = acc[i][2 * q + 1] * inv;
                if (a.gain2) {
                    y0 *= elem(nv2[i], 2 * q);
                    y1 *= elem(nv2[i], 2 * q + 1);
                }
                o[q] = pack_bf16x2(y0, y1);
            }
            store_out_vec(out2_row, (uint32_t)st(i) * 16u, o);
        }
        return;
    }

    if constexpr (kNorm) {
        // Effective per-element weight.
        float g[VPT][8];
#pragma unroll
        for (int i = 0; i < VPT; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (EPI == Epilogue::kBeamNorm)
                    g[i][e] = a.gain ? elem(gv[i], e) : 1.0f;
                else
                    g[i][e] = elem(gv[i], e) + a.gain_center;
            }
        if constexpr (EPI == Epilogue::kRmsNormWeightFirst) {
#pragma unroll
            for (int i = 0; i < VPT; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[i][e] *= g[i][e];
        }
        const float ss = row_sum_sq<VPT, TPW>(acc);
        const float inv = rsqrtf(ss / (float)a.hidden + a.eps);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                y[e] = acc[i][e] * inv;
                if constexpr (EPI != Epilogue::kRmsNormWeightFirst)
                    y[e] *= g[i][e];
            }
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                o[q] = pack_bf16x2(y[2 * q], y[2 * q + 1]);
            store(i, o);
        }
    }
}

// One workgroup finalizes token a.token_base + blockIdx.x (TPW > 1: the
// TPW tokens of a token block, described below).
//   L      where slot rows come from (index map, token major, one row per token)
//   W_BF16 weights are BF16 (else FP32)
//   EPI    what follows the FP32 routed sum
//   KC     top_k when known at compile time (> 0), else minus the largest
//          top-k the kernel serves (a.top_k is read at run time)
//   VPT    16-byte vectors per thread; EXACT: hidden / 8 == blockDim.x * VPT
//
// Slots whose rows all fit in flight (slots_in_flight) arrive as one batch:
// every valid slot's row vectors are issued, then the FMAs run.  More slots
// than that stream through a rolling window of W slots: the rows of slot
// s + W are issued as soon as slot s has been reduced, so a token's loads
// never drain between groups of slots.  The window's code is straight-line:
// its loads go through buffer resources, and an invalid slot, or one past a
// run-time top-k, gets an empty resource whose loads return zeros without
// touching memory, and weight 0.  Every load is then unconditional, the
// compiler waits for exactly the slot being reduced, and a scheduling
// barrier per slot keeps each slot's loads W slots ahead of its FMAs instead
// of all at the top.  fma(0, 0, acc) == acc bit for bit, since a sum that
// starts at +0 never becomes -0.
//
// TPW > 1 (hidden 256, whose 32 vectors fill half a wave, up to top-k 7;
// hidden 512 at top-k 1): a one-wave workgroup finalizes TPW consecutive
// tokens of the launch, 64 / TPW lanes each, VPT = hidden / 8 / (64 / TPW)
// vectors per lane; their output rows are adjacent, so one resource spans
// them all.  Tokens past the last gather nothing and their stores fall
// outside that resource.
template <Layout L, bool W_BF16, Epilogue EPI, int KC, int VPT, bool EXACT, int TPW>
__global__ void __launch_bounds__(TPW > 1 ? kWave : max_team(VPT))
finalize_kernel(const FinalizeArgs a)
{
    constexpr bool kIdx = L == Layout::kIndexMap;
    static_assert(TPW == 1 || (EXACT && ((VPT * kWave == 32 * TPW && wave_tokens(KC) == TPW) ||
                                         (VPT * kWave == 64 * TPW && KC == 1 && TPW == 2))),
                  "TPW tokens of 32 vectors (hidden 256) or two of 64 (hidden 512) in one wave");
    constexpr int KB = TPW > 1 ? (KC > 0 ? KC : -KC) : slots_in_flight(kIdx, KC, VPT);
    constexpr bool kRoll = TPW == 1 && rolling(kIdx, KC, VPT);
    constexpr int kSlotsMax = KC > 0 ? KC : -KC;
    static_assert(KB >= 1 && (kRoll || KC <= 0 || KC % KB == 0), "batches divide top-k");
    constexpr bool kNorm = EPI == Epilogue::kRmsNorm || EPI == Epilogue::kRmsNormWeightFirst ||
                           EPI == Epilogue::kBeamNorm;
    // Lanes per token; with TPW > 1, lane l holds vectors l % LPT + LPT i of
    // token l / LPT.
    constexpr int LPT = kWave / TPW;
    const int top_k = KC > 0 ? KC : a.top_k;
    const int team = blockDim.x;
    const int lane = threadIdx.x;
    const int nv = a.hidden >> 3;
    // The workgroup's first token and how many of its TPW tokens exist.
    // Multi-token waves read 4-16 bytes of slot metadata per token, so one
    // cache line holds that of 8 or more workgroups: runs of consecutive
    // token blocks go to one XCD (its own L2), which would otherwise fetch
    // each line on all 8 (measured at top-k 1: 11 % more bytes read than
    // the method moves on the index map, 5 % token major).
    const unsigned blk = TPW > 1 ? xcd_run_block(blockIdx.x, gridDim.x, MF_XCD_RUN) : blockIdx.x;
    const int64_t t0 = a.token_base + (int64_t)blk * TPW;
    const int n_live = TPW == 1 || t0 + TPW <= a.num_tokens ? TPW : (int)(a.num_tokens - t0);
    const int64_t t = t0;
    const int64_t tk = t * top_k;
    auto col = [&](int i) { return TPW > 1 ? lane % LPT + LPT * i : lane + i * team; };

    // The norm weight is shared by every token and stays cache resident;
    // fetch it first so its latency hides under the gather.  A multi-token
    // wave reads an optional weight through a resource that is empty when
    // the weight is absent: under a branch, the register copy that joins
    // the two paths waits for the load before the first gather, which a
    // wave of one-slot tokens, its whole life two round trips, cannot hide.
    u32x4 gv[VPT];
    if constexpr (kNorm || EPI == Epilogue::kResidualNorm) {
        const bool have = (EPI != Epilogue::kBeamNorm && EPI != Epilogue::kResidualNorm) ||
                          a.gain != nullptr;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int j = col(i);
            gv[i] = (u32x4){0u, 0u, 0u, 0u};
            if constexpr (TPW > 1)
                gv[i] = load_vec_bounded<0>(a.gain, have ? nv : 0, j);
            else if (have)
                gv[i] = EXACT ? reinterpret_cast<const u32x4 *>(a.gain)[j]
                              : load_vec_bounded<0>(a.gain, nv, j);
        }
    }

    // The residual row of this token, for the residual epilogue.
    u32x4 rv[VPT];
    if constexpr (EPI == Epilogue::kResidualNorm) {
        const u32x4 *rr = reinterpret_cast<const u32x4 *>(a.residual + t * (int64_t)a.hidden);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int j = col(i);
            if constexpr (TPW > 1)   // the workgroup's rows are adjacent
                rv[i] = load_vec_bounded<MF_ROW_LOAD_POLICY>(rr, n_live * nv, lane / LPT * nv + j);
            else
                rv[i] = EXACT ? load_row_vec(rr + j)
                              : load_vec_bounded<MF_ROW_LOAD_POLICY>(rr, nv, j);
        }
    }

    // A direct row starts from -0, so that fma(1, x, -0) == x for every x,
    // -0 included; a routed sum starts from +0.
    constexpr float kAcc0 = L == Layout::kDirect ? -0.0f : 0.0f;
    float acc[VPT][8];
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[i][e] = kAcc0;

    if constexpr (kRoll) {
        constexpr int W = KB < kSlotsMax ? KB : kSlotsMax;
        // Slot metadata in VGPRs: lane l of every wave holds slot l's index
        // and weight (lanes past top-k an invalid index and weight 0), read
        // back as scalars per slot.  The loads are unconditional: lanes past
        // top-k re-read the last slot.
        const int wl = lane & (kWave - 1);
        const int64_t ms = tk + (wl < top_k ? wl : top_k - 1);
        int32_t m_idx = -1;
        if constexpr (kIdx)
            m_idx = a.idx[ms];
        float m_w = load_weight<W_BF16>(a.weights, ms);
        if (wl >= top_k) {
            m_idx = -1;
            m_w = 0.0f;
        }

        u32x4 v[W][VPT];
        float wt[W];
        // The row address is computed whether or not the slot is valid (an
        // empty resource never dereferences it): a select between it and a
        // constant would be turned into a branch, and branches between the
        // slots would let the compiler sink each slot's FMAs past the loads
        // that follow them.
        const uint64_t rows = reinterpret_cast<uintptr_t>(a.rows);
        auto issue = [&](int s) {
            const int b = s % W;
            const float w = lane_value(m_w, s);
            bool ok;
            int64_t off;   // elements
            if constexpr (kIdx) {
                const int32_t i = lane_value(m_idx, s);
                ok = i >= 0 && (int64_t)i < a.num_rows;
                off = (int64_t)i * a.row_stride;
            } else {
                ok = KC > 0 || s < top_k;
                off = (tk + s) * (int64_t)a.hidden;
            }
            wt[b] = ok ? w : 0.0f;
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                reinterpret_cast<void *>(rows + 2 * (uint64_t)off), 0, ok ? nv * 16 : 0,
                kRawBufferWord3);
#pragma unroll
            for (int i = 0; i < VPT; ++i)   // vectors past the row read as zeros
                v[b][i] = __builtin_amdgcn_raw_buffer_load_b128(r, (lane + i * team) * 16, 0,
                                                                MF_ROW_LOAD_POLICY);
        };
#pragma unroll
        for (int s = 0; s < W; ++s)
            issue(s);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < kSlotsMax; ++s) {
            const int b = s % W;
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[i][e] = __builtin_fmaf(wt[b], elem(v[b][i], e), acc[i][e]);
                // An empty statement that reads and writes the sums keeps this
                // slot's FMAs here: otherwise instruction selection may place
                // every slot's FMAs after the last barrier, with all 32 slots'
                // rows held in registers.
                asm volatile("" : "+v"(acc[i][0]), "+v"(acc[i][1]), "+v"(acc[i][2]),
                             "+v"(acc[i][3]), "+v"(acc[i][4]), "+v"(acc[i][5]),
                             "+v"(acc[i][6]), "+v"(acc[i][7]));
            }
            if (s + W < kSlotsMax)
                issue(s + W);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else if constexpr (TPW > 1) {
        // Every lane gathers its own token's rows through a per-lane
        // address.  Slot metadata is uniform per token (scalar loads) and
        // each lane picks its token's.  Three phases, in this order so that
        // no wait stands between the row loads and their issue: the index
        // map's row indices; every row load; the weights.  A lane whose slot
        // is invalid or past a run-time top-k, or whose token is past the
        // last, reads the zero row instead, with weight 0, so every load is
        // unconditional.  A dead token's metadata reads are those of t0.
        const int q = lane / LPT;
        const bool live_q = q < n_live;
        auto slot = [&](int u, int k) {   // metadata position of token t0 + u, slot k
            const int64_t tu = u < n_live ? t0 + u : t0;
            return tu * top_k + (KC > 0 ? k : (k < top_k ? k : top_k - 1));
        };
        // Each lane keeps its own token's value as the uniform values of the
        // TPW tokens arrive (selected into a register, never an array the
        // compiler could place in LDS).
        int32_t ik[kSlotsMax] = {};
        if constexpr (kIdx) {
#pragma unroll
            for (int k = 0; k < kSlotsMax; ++k)
#pragma unroll
                for (int u = 0; u < TPW; ++u) {
                    const int32_t x = a.idx[slot(u, k)];
                    ik[k] = u == 0 || q == u ? x : ik[k];
                }
        }
        const int64_t tq = live_q ? t0 + q : t0;
        bool ok[kSlotsMax];
        u32x4 v[kSlotsMax][VPT];
#pragma unroll
        for (int k = 0; k < kSlotsMax; ++k) {
            ok[k] = live_q && (KC > 0 || k < top_k);
            int64_t off;   // elements
            if constexpr (kIdx) {
                ok[k] = ok[k] && ik[k] >= 0 && (int64_t)ik[k] < a.num_rows;
                off = (int64_t)ik[k] * a.row_stride;
            } else if constexpr (L == Layout::kTokenMajor) {
                off = (tq * top_k + k) * (int64_t)a.hidden;
            } else {   // kDirect
                off = tq * a.row_stride;
            }
            const u32x4 *src =
                (ok[k] ? reinterpret_cast<const u32x4 *>(a.rows + off) : zero_row) + lane % LPT;
#pragma unroll
            for (int i = 0; i < VPT; ++i)
                v[k][i] = load_row_vec(src + LPT * i);
        }
        __builtin_amdgcn_sched_barrier(0);
        float w[kSlotsMax];
#pragma unroll
        for (int k = 0; k < kSlotsMax; ++k) {
            w[k] = 1.0f;
            if constexpr (L != Layout::kDirect)
#pragma unroll
                for (int u = 0; u < TPW; ++u) {
                    const float x = load_weight<W_BF16>(a.weights, slot(u, k));
                    w[k] = u == 0 || q == u ? x : w[k];
                }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < kSlotsMax; ++k)
            w[k] = ok[k] ? w[k] : 0.0f;
#pragma unroll
        for (int k = 0; k < kSlotsMax; ++k)
#pragma unroll
            for (int i = 0; i < VPT; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[i][e] = __builtin_fmaf(w[k], elem(v[k][i], e), acc[i][e]);
    } else {
        // Batches of KB slots (one batch when every slot fits): uniform
        // per-slot data first (scalar loads, one wait), then every valid
        // slot's row vectors, then the FMAs in ascending slot order.  The
        // batches are unrolled up to the slots the kernel serves, with a
        // uniform exit past a run-time top-k.
#pragma unroll
        for (int k0 = 0; k0 < kSlotsMax; k0 += KB) {
            if (KC < 0 && k0 >= top_k)
                break;
            int64_t row_off[KB];   // elements
            bool ok[KB];
            float w[KB];
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                // Slots past a run-time top-k re-read the token's last slot
                // (always in bounds) and are masked: the metadata loads stay
                // unconditional, so they issue together behind one wait.
                const int k = k0 + b;
                const bool live = KC > 0 || k < top_k;
                const int kk = KC > 0 ? k : (k < top_k ? k : top_k - 1);
                if constexpr (kIdx) {
                    w[b] = load_weight<W_BF16>(a.weights, tk + kk);
                    const int32_t i = a.idx[tk + kk];
                    ok[b] = live && i >= 0 && (int64_t)i < a.num_rows;
                    row_off[b] = (int64_t)i * a.row_stride;
                } else if constexpr (L == Layout::kTokenMajor) {
                    w[b] = load_weight<W_BF16>(a.weights, tk + kk);
                    ok[b] = live;
                    row_off[b] = (tk + kk) * (int64_t)a.hidden;
                } else {   // kDirect
                    w[b] = 1.0f;
                    ok[b] = live;
                    row_off[b] = t * a.row_stride;
                }
            }
            u32x4 v[KB][VPT];
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                if (ok[b]) {
                    const u32x4 *r = reinterpret_cast<const u32x4 *>(a.rows + row_off[b]);
#pragma unroll
                    for (int i = 0; i < VPT; ++i) {
                        const int j = lane + i * team;
                        v[b][i] = EXACT ? load_row_vec(r + j)
                                        : load_vec_bounded<MF_ROW_LOAD_POLICY>(r, nv, j);
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                if (ok[b]) {
#pragma unroll
                    for (int i = 0; i < VPT; ++i)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[i][e] = __builtin_fmaf(w[b], elem(v[b][i], e), acc[i][e]);
                }
            }
            // Every gather of this batch has been consumed.  Saying so keeps
            // the compiler, which cannot pair each conditional load with its
            // conditional use, from waiting before each gather of the next
            // batch.
            if constexpr (kSlotsMax > KB)
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        }
    }

    // The workgroup's output rows are adjacent: one resource spans those of
    // its live tokens.
    finish_token<EPI, VPT, EXACT, TPW>(acc, gv, rv, a, t0, n_live * nv, lane, team);
}

// ------------------------------------------------------------ dispatch ---

// The current device's LDS per CU and per workgroup and its CU count,
// queried once per device (concurrent first calls store the same values);
// all zero if a query fails, and then no residency cap applies.
struct DeviceLimits {
    int lds_per_cu, lds_per_block, cus;
};

DeviceLimits device_limits()
{
    static std::atomic<int> cached[64][3];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return DeviceLimits{};
    DeviceLimits d{cached[dev][0].load(std::memory_order_relaxed),
                   cached[dev][1].load(std::memory_order_relaxed),
                   cached[dev][2].load(std::memory_order_relaxed)};
    if (d.lds_per_cu > 0 && d.lds_per_block > 0 && d.cus > 0)
        return d;
    if (hipDeviceGetAttribute(&d.lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              dev) != hipSuccess ||
        hipDeviceGetAttribute(&d.lds_per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess ||
        hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        d.lds_per_cu <= 0 || d.lds_per_block <= 0 || d.cus <= 0)
        return DeviceLimits{};
    cached[dev][0].store(d.lds_per_cu, std::memory_order_relaxed);
    cached[dev][1].store(d.lds_per_block, std::memory_order_relaxed);
    cached[dev][2].store(d.cus, std::memory_order_relaxed);
    return d;
}

// Launch the kernel of plan p over all tokens, at most p.max_tokens per
// launch (each launch starts at its token_base), with the dynamic LDS that
// sets the workgroups resident per CU (plan.hpp).
template <Layout L, bool W_BF16, Epilogue EPI, int KC>
hipError_t launch_plan(const FinalizeArgs &a, const LaunchPlan &p, hipStream_t s)
{
    const DeviceLimits d = device_limits();
    // A workgroup's rows in flight cover its p.tpw tokens.
    const int64_t workgroups = (a.num_tokens + p.tpw - 1) / p.tpw;
    const int64_t blocks = residency_blocks(L == Layout::kIndexMap, a.hidden * p.tpw, p.slots,
                                            workgroups, d.cus);
    const size_t lds =
        (size_t)residency_lds(blocks, d.lds_per_cu, d.lds_per_block, kStaticLds);
    FinalizeArgs c = a;
    for (int64_t t0 = 0; t0 < a.num_tokens; t0 += p.max_tokens) {
        c.token_base = t0;
        const int64_t count = std::min<int64_t>(p.max_tokens, a.num_tokens - t0);
        const dim3 grid((unsigned)((count + p.tpw - 1) / p.tpw));
        const dim3 block((unsigned)p.team);
        if constexpr (wave_tokens(KC) > 1) {
            if (p.tpw == wave_tokens(KC) && p.vpt == wave_tokens(KC) / 2) {   // hidden 256
                hipLaunchKernelGGL((finalize_kernel<L, W_BF16, EPI, KC, wave_tokens(KC) / 2, true,
                                                    wave_tokens(KC)>),
                                   grid, block, lds, s, c);
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess)
                    return e;
                continue;
            }
        }
        if constexpr (KC == 1 && MF_WAVE_TOKENS_512) {
            if (p.tpw == 2 && p.vpt == 2) {   // hidden 512, two tokens per wave
                hipLaunchKernelGGL((finalize_kernel<L, W_BF16, EPI, 1, 2, true, 2>), grid, block,
                                   lds, s, c);
                const hipError_t e = hipGetLastError();
                if (e != hipSuccess)
                    return e;
                continue;
            }
        }
        // A routed call reaches slot count 1 only at hidden 256 and 512,
        // whose multi-token kernels ran above: no one-token kernel exists
        // for it.
        if constexpr (KC == 1 && L != Layout::kDirect)
            return hipErrorInvalidValue;
        switch (p.vpt) {
        case 8:
            if constexpr (vpt_possible(L == Layout::kIndexMap, KC, 8))
                hipLaunchKernelGGL((finalize_kernel<L, W_BF16, EPI, KC, 8, true, 1>), grid, block,
                                   lds, s, c);
            break;
        case 4:
            if constexpr (vpt_possible(L == Layout::kIndexMap, KC, 4))
                hipLaunchKernelGGL((finalize_kernel<L, W_BF16, EPI, KC, 4, true, 1>), grid, block,
                                   lds, s, c);
            break;
        case 2:
            if constexpr (vpt_possible(L == Layout::kIndexMap, KC, 2))
                hipLaunchKernelGGL((finalize_kernel<L, W_BF16, EPI, KC, 2, true, 1>), grid, block,
                                   lds, s, c);
            break;
        case 1:
            if constexpr (vpt_possible(L == Layout::kIndexMap, KC, 1))
                hipLaunchKernelGGL((finalize_kernel<L, W_BF16, EPI, KC, 1, true, 1>), grid, block,
                                   lds, s, c);
            break;
        default:   // n odd: 32 (n + 1) threads, the last half wave idle
            if constexpr (vpt_possible(L == Layout::kIndexMap, KC, 0))
                hipLaunchKernelGGL((finalize_kernel<L, W_BF16, EPI, KC, 1, false, 1>), grid, block,
                                   lds, s, c);
            break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// Compile-time slot counts for the common top-k values (8, 16); other top-k
// are read at run time by kernels sized for 2, 4, 8, 12, 16, 24 or 32 slots.
template <Layout L, bool W_BF16, Epilogue EPI>
hipError_t launch_topk(const FinalizeArgs &a, hipStream_t s)
{
    const LaunchPlan p = plan_launch(L == Layout::kIndexMap, false, a.hidden, a.top_k);
    switch (p.kc) {
    case 1:   // top-k 1 at hidden 256 and 512: several tokens per wave
        if constexpr (wave_tokens(1) > 1 || MF_WAVE_TOKENS_512)
            return launch_plan<L, W_BF16, EPI, 1>(a, p, s);
        return hipErrorInvalidValue;
    case 8:
        return launch_plan<L, W_BF16, EPI, 8>(a, p, s);
    case 16:
        return launch_plan<L, W_BF16, EPI, 16>(a, p, s);
    case -2:
        return launch_plan<L, W_BF16, EPI, -2>(a, p, s);
    case -4:
        return launch_plan<L, W_BF16, EPI, -4>(a, p, s);
    case -8:
        return launch_plan<L, W_BF16, EPI, -8>(a, p, s);
    case -12:
        return launch_plan<L, W_BF16, EPI, -12>(a, p, s);
    case -16:
        return launch_plan<L, W_BF16, EPI, -16>(a, p, s);
    case -24:
        return launch_plan<L, W_BF16, EPI, -24>(a, p, s);
    case -32:
        return launch_plan<L, W_BF16, EPI, -32>(a, p, s);
    default:
        return hipErrorInvalidValue;
    }
}

template <Epilogue EPI>
hipError_t launch_index_map(const FinalizeArgs &a, hipStream_t s)
{
    return a.weights_bf16 ? launch_topk<Layout::kIndexMap, true, EPI>(a, s)
                          : launch_topk<Layout::kIndexMap, false, EPI>(a, s);
}

template <Epilogue EPI>
hipError_t launch_direct(const FinalizeArgs &a, hipStream_t s)
{
    return launch_plan<Layout::kDirect, false, EPI, 1>(
        a, plan_launch(false, true, a.hidden, 1), s);
}

hipError_t dispatch(const FinalizeArgs &a, Layout layout, Epilogue epi, hipStream_t s)
{
    if (a.top_k < 1 || a.top_k > kMaxTopK || a.num_tokens < 0)
        return hipErrorInvalidValue;
    switch (layout) {
    case Layout::kIndexMap:
        switch (epi) {
        case Epilogue::kRound:
            return launch_index_map<Epilogue::kRound>(a, s);
        case Epilogue::kRmsNorm:
            return launch_index_map<Epilogue::kRmsNorm>(a, s);
        case Epilogue::kRmsNormWeightFirst:
            return launch_index_map<Epilogue::kRmsNormWeightFirst>(a, s);
        default:
            break;
        }
        break;
    case Layout::kTokenMajor:
        switch (epi) {
        case Epilogue::kBeam:
            return launch_topk<Layout::kTokenMajor, false, Epilogue::kBeam>(a, s);
        case Epilogue::kBeamNorm:
            return launch_topk<Layout::kTokenMajor, false, Epilogue::kBeamNorm>(a, s);
        case Epilogue::kResidualNorm:
            return launch_topk<Layout::kTokenMajor, false, Epilogue::kResidualNorm>(a, s);
        default:
            break;
        }
        break;
    case Layout::kDirect:
        switch (epi) {
        case Epilogue::kRmsNorm:
            return launch_direct<Epilogue::kRmsNorm>(a, s);
        case Epilogue::kRmsNormWeightFirst:
            return launch_direct<Epilogue::kRmsNormWeightFirst>(a, s);
        case Epilogue::kResidualNorm:
            return launch_direct<Epilogue::kResidualNorm>(a, s);
        default:
            break;
        }
        break;
    }
    return hipErrorInvalidValue;
}

}  // namespace

int launch_finalize(const FinalizeArgs &a, Layout layout, Epilogue epi, void *stream)
{
    return static_cast<int>(dispatch(a, layout, epi, static_cast<hipStream_t>(stream)));
}

const char *launch_error_string(int code)
{
    return hipGetErrorString(static_cast<hipError_t>(code));
}

}  // namespace mf
