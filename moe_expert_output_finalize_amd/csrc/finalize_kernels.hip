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
//  - the token's indices and weights are uniform, so they live in SGPRs and
//    validity is a scalar branch: invalid slots issue no memory traffic;
//  - up to 16 row vectors per thread are in flight before the first FMA:
//    all of a token's rows at top-k 8, and at top-k 16 with one vector per
//    thread (index map up to hidden 4096); larger top-k in batches;
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

#include "launch.hpp"

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
#ifndef MF_INFLIGHT_KB_PER_CU
#define MF_INFLIGHT_KB_PER_CU 128 // > 0: cap resident workgroups so that their row
                                  // loads in flight total about this much per CU
#endif
// Row vectors in flight per thread.  16 (64 VGPRs) keeps two workgroups per
// CU at two vectors per thread; 32 had let an index-map top-k 16 token have
// all its rows in flight, but at hidden above 4096 the 150-160 VGPRs that
// takes leave one workgroup per CU (hidden 5120-8192, top-k 12-16: 3-11 %
// slower than batches of 8).  A token-major token is one contiguous block,
// also faster fetched in halves (top-k 16: 10 % faster than all at once).
#ifndef MF_MAX_VECS_INDEX_MAP
#define MF_MAX_VECS_INDEX_MAP 16
#endif
#ifndef MF_MAX_VECS_TOKEN_MAJOR
#define MF_MAX_VECS_TOKEN_MAJOR 16
#endif
#ifndef MF_VPT_ORDER
#define MF_VPT_ORDER 2, 1, 4, 8 // preferred vectors per thread, first that fits
#endif
// Index-map rows up to this hidden size take one vector per thread instead
// (teams of up to 512 threads): 1 % faster at 8192 tokens and hidden 4096,
// 5 % at 256 tokens, 3 % at hidden 2048 / top-k 16; at hidden 7168 the
// 896-thread teams are 5 % slower, and token-major tokens prefer two
// vectors per thread at every size measured.  0 disables the override.
#ifndef MF_INDEX_MAP_VPT1_MAX_HIDDEN
#define MF_INDEX_MAP_VPT1_MAX_HIDDEN 4096
#endif

namespace mf {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxTopK = 32;   // the entry points reject larger top-k
// s_waitcnt operand on gfx9: vmcnt(0), expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kMaxWaves = 16;

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

// ------------------------------------------------------------ memory -----

__device__ __forceinline__ u32x4 load_row_vec(const u32x4 *p)
{
#if MF_NONTEMPORAL_ROWS
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

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

// Sum of v over the workgroup, returned to every thread.  All threads of the
// workgroup must call it (it contains a barrier when there are several waves).
// Two sums in one kernel use different banks, so the second's LDS writes
// cannot overtake a slower wave's reads of the first.
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

// ------------------------------------------------------------ kernel -----

// Row vectors one thread keeps in flight.  One vector per thread means teams
// of up to 1024 threads, whose launch bound leaves 128 VGPRs per thread: at
// most 16 vectors (64 VGPRs) there.
constexpr int max_vecs(Layout l, int vpt)
{
    const int m = l == Layout::kIndexMap ? MF_MAX_VECS_INDEX_MAP : MF_MAX_VECS_TOKEN_MAJOR;
    return vpt == 1 && m > 16 ? 16 : m;
}

// Slot-count template argument for a top-k read at run time:
//   KC > 0   top-k is KC;
//   KC == 0  any top-k, in batches of max_vecs / VPT slots;
//   KC < 0   top-k at most -KC, registers sized for -KC slots, so a small
//            top-k keeps a small register footprint and high occupancy.
constexpr int small_topk_kc(int top_k) { return top_k <= 2 ? -2 : top_k <= 4 ? -4 : -8; }

// Slots whose rows one workgroup has in flight at once: all of them when
// they fit, else batches of max_vecs / VPT; a run-time top-k above 8 at one
// vector per thread takes batches of 12, which keeps its unrolled batches
// within the 128 VGPRs of a 1024-thread launch bound without spilling.
constexpr int slots_in_flight(Layout l, int kc, int vpt)
{
    const int want = kc < 0 ? -kc : kc;
    if (kc == 0 && vpt == 1)
        return max_vecs(l, vpt) < 12 ? max_vecs(l, vpt) : 12;
    return (want > 0 && want * vpt <= max_vecs(l, vpt)) ? want : max_vecs(l, vpt) / vpt;
}

template <int VPT>
constexpr int max_team() { return VPT == 1 ? 1024 : VPT == 2 ? 512 : 256; }

// One workgroup finalizes token blockIdx.x.
//   L      where slot rows come from (index map, token major, one row per token)
//   W_BF16 weights are BF16 (else FP32)
//   EPI    what follows the FP32 routed sum
//   KC     top_k when known at compile time (0: read a.top_k; negative: read
//          a.top_k, which is at most -KC)
//   VPT    16-byte vectors per thread; EXACT: hidden / 8 == blockDim.x * VPT
template <Layout L, bool W_BF16, Epilogue EPI, int KC, int VPT, bool EXACT>
__global__ void __launch_bounds__(max_team<VPT>())
finalize_kernel(const FinalizeArgs a)
{
    constexpr int KB = slots_in_flight(L, KC, VPT);
    static_assert(KB >= 1 && (KC <= 0 || KC % KB == 0), "slot batch must divide top_k");
    constexpr bool kNorm = EPI == Epilogue::kRmsNorm || EPI == Epilogue::kRmsNormWeightFirst ||
                           EPI == Epilogue::kBeamNorm;
    constexpr bool kBeamRounding = EPI == Epilogue::kBeam || EPI == Epilogue::kBeamNorm ||
                                   EPI == Epilogue::kResidualNorm;
    const int top_k = KC > 0 ? KC : a.top_k;
    const int team = blockDim.x;
    const int lane = threadIdx.x;
    const int nv = a.hidden >> 3;
    const int64_t t = blockIdx.x;
    const int64_t tk = t * top_k;

    // The norm weight is shared by every token and stays cache resident;
    // fetch it first so its latency hides under the gather.
    u32x4 gv[VPT];
    if constexpr (kNorm || EPI == Epilogue::kResidualNorm) {
        const bool have = (EPI != Epilogue::kBeamNorm && EPI != Epilogue::kResidualNorm) ||
                          a.gain != nullptr;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int j = lane + i * team;
            gv[i] = (u32x4){0u, 0u, 0u, 0u};
            if (have && (EXACT || j < nv))
                gv[i] = reinterpret_cast<const u32x4 *>(a.gain)[j];
        }
    }

    // The residual row of this token, for the residual epilogue.
    u32x4 rv[VPT];
    if constexpr (EPI == Epilogue::kResidualNorm) {
        const u32x4 *rr = reinterpret_cast<const u32x4 *>(a.residual + t * (int64_t)a.hidden);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int j = lane + i * team;
            rv[i] = (u32x4){0u, 0u, 0u, 0u};
            if (EXACT || j < nv)
                rv[i] = load_row_vec(rr + j);
        }
    }

    float acc[VPT][8];
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[i][e] = 0.0f;

    // Batches are unrolled up to the largest top-k the entry points accept,
    // with a uniform exit: a loop with a run-time trip count makes the
    // compiler wait for every earlier load before each gather.
    constexpr int kSlotsMax = KC > 0 ? KC : KC < 0 ? -KC : kMaxTopK;
#pragma unroll
    for (int k0 = 0; k0 < kSlotsMax; k0 += KB) {
        if (KC <= 0 && k0 >= top_k)
            break;
        // Uniform per-slot data first (scalar loads, one wait), then every
        // valid slot's row vectors, then the FMAs in ascending slot order.
        int64_t row_off[KB];   // elements
        bool ok[KB];
        float w[KB];
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            const int k = k0 + b;
            // Slots past a run-time top-k re-read the token's last slot
            // (always in bounds) and are masked: the metadata loads stay
            // unconditional, so they issue together behind one wait.
            const bool live = KC > 0 || k < top_k;
            const int kk = KC > 0 ? k : (k < top_k ? k : top_k - 1);
            if constexpr (L == Layout::kIndexMap) {
                w[b] = load_weight<W_BF16>(a.weights, tk + kk);
                const int32_t i = a.idx[tk + kk];
                ok[b] = live && i >= 0 && (int64_t)i < a.num_rows;
                row_off[b] = (int64_t)i * a.row_stride;
            } else if constexpr (L == Layout::kTokenMajor) {
                w[b] = load_weight<W_BF16>(a.weights, tk + kk);
                ok[b] = live;
                row_off[b] = (tk + kk) * (int64_t)a.hidden;
            } else {   // kDirect: fma(1, x, +0) == x exactly
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
                    if (EXACT || j < nv)
                        v[b][i] = load_row_vec(r + j);
                    else
                        v[b][i] = (u32x4){0u, 0u, 0u, 0u};
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
        // Every gather of this batch has been consumed.  Saying so keeps the
        // compiler, which cannot pair each conditional load with its
        // conditional use, from waiting before each gather of the next batch.
        if constexpr (kSlotsMax > KB)
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }

    const __amdgpu_buffer_rsrc_t out_row =
        row_resource(a.out + t * (int64_t)a.hidden, (uint32_t)nv * 16u);
    auto store = [&](int i, const u32x4 &o) {
        const int j = lane + i * team;
        if (EXACT || j < nv)
            store_out_vec(out_row, (uint32_t)j * 16u, o);
    };

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
            float ss = 0.0f;
#pragma unroll
            for (int i = 0; i < VPT; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    ss = __builtin_fmaf(acc[i][e], acc[i][e], ss);
            ss = block_sum(ss, 0);
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
        // hidden = bf16(scale_x * y + scale_res * residual), kept widened in acc.
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float h0 = __builtin_fmaf(a.scale_x, acc[i][2 * q],
                                                a.scale_res * elem(rv[i], 2 * q));
                const float h1 = __builtin_fmaf(a.scale_x, acc[i][2 * q + 1],
                                                a.scale_res * elem(rv[i], 2 * q + 1));
                const uint32_t p = pack_bf16x2(h0, h1);
                o[q] = p;
                acc[i][2 * q] = bf16_lo(p);
                acc[i][2 * q + 1] = bf16_hi(p);
            }
            store(i, o);
        }
        if (!a.has_next)
            return;
        // normalized = bf16(hidden * inv_rms(hidden) * next_weight)
        u32x4 nv2[VPT];
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int j = lane + i * team;
            nv2[i] = (u32x4){0u, 0u, 0u, 0u};
            if (a.gain2 && (EXACT || j < nv))
                nv2[i] = reinterpret_cast<const u32x4 *>(a.gain2)[j];
        }
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < VPT; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                ss = __builtin_fmaf(acc[i][e], acc[i][e], ss);
        ss = block_sum(ss, 1);
        const float inv = rsqrtf(ss / (float)a.hidden + a.eps2);
        const __amdgpu_buffer_rsrc_t out2_row =
            row_resource(a.out2 + t * (int64_t)a.hidden, (uint32_t)nv * 16u);
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
            const int j = lane + i * team;
            if (EXACT || j < nv)
                store_out_vec(out2_row, (uint32_t)j * 16u, o);
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
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < VPT; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                ss = __builtin_fmaf(acc[i][e], acc[i][e], ss);   // idle vectors hold 0
        ss = block_sum(ss);
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

// ------------------------------------------------------------ dispatch ---

// Whether `vpt` can be chosen at all: once a value that fits every even n
// (VPT 1) appears in MF_VPT_ORDER, later entries are never picked, so their
// kernels are not instantiated.
constexpr bool vpt_reachable(int vpt)
{
    constexpr int order[] = {MF_VPT_ORDER};
    for (int v : order) {
        if (v == vpt)
            return true;
        if (v == 1)
            return false;
    }
    return false;
}

// Whether a team of 32 n / vpt threads is a whole number of waves within the
// launch bound of that vpt.
inline bool team_fits(int n, int vpt)
{
    const int team = 32 * n / vpt;
    const int bound = vpt == 1 ? 1024 : vpt == 2 ? 512 : 256;
    return (32 * n) % vpt == 0 && team % kWave == 0 && team >= kWave && team <= bound;
}

// Vectors per thread for hidden = 256 n: one for index-map rows up to
// MF_INDEX_MAP_VPT1_MAX_HIDDEN, else the first of MF_VPT_ORDER whose team
// fits; 0 if none (then one vector per thread with the last half wave idle).
// On the index map, a run-time top-k below 8 (kc < 0) widens that by
// 8 / -kc where the team still fits, so a thread keeps about as many row
// vectors in flight as at top-k 8 while workgroups stay small enough for
// high occupancy (2-8 % faster at top-k 2 and 4; token-major rows measured
// faster without it).
inline int pick_vpt(Layout l, int n, int kc)
{
    int base = 0;
    if (l == Layout::kIndexMap && 256 * n <= MF_INDEX_MAP_VPT1_MAX_HIDDEN && n % 2 == 0 &&
        vpt_reachable(1)) {
        base = 1;
    } else {
        for (int vpt : {MF_VPT_ORDER})
            if (team_fits(n, vpt)) {
                base = vpt;
                break;
            }
    }
    if (l == Layout::kIndexMap && kc < 0 && base > 0)
        for (int vpt = std::min(8, base * 8 / -kc); vpt > base; vpt /= 2)
            if (team_fits(n, vpt))
                return vpt;
    return base;
}

// Dynamic LDS to reserve per workgroup so that a CU holds
// ceil(MF_INFLIGHT_KB_PER_CU / in-flight bytes per workgroup) workgroups,
// clamped to 2..16.  Beyond that, extra concurrent gathers do not raise
// bandwidth; they stretch every token's lifetime and with it the tail of
// the launch (measured: 2-5 % faster on every large workload than residency
// limited by registers).  The kernels' own LDS use is 64 bytes.
inline size_t residency_lds(int hidden, int slots)
{
#if MF_INFLIGHT_KB_PER_CU > 0
    // Per-device LDS limits, queried once; concurrent first calls store the
    // same values.
    static std::atomic<int> lds_per_cu[64], lds_per_block[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 0;
    int cu = lds_per_cu[dev].load(std::memory_order_relaxed);
    int blk = lds_per_block[dev].load(std::memory_order_relaxed);
    if (cu <= 0 || blk <= 0) {
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
                hipSuccess ||
            hipDeviceGetAttribute(&blk, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
                hipSuccess || cu <= 0 || blk <= 0)
            return 0;
        lds_per_cu[dev].store(cu, std::memory_order_relaxed);
        lds_per_block[dev].store(blk, std::memory_order_relaxed);
    }
    const int64_t per_block = 2LL * hidden * slots;           // row bytes in flight
    const int64_t want = ((int64_t)MF_INFLIGHT_KB_PER_CU * 1024 + per_block - 1) / per_block;
    const int64_t blocks = std::min<int64_t>(16, std::max<int64_t>(2, want));
    const int64_t lds = std::min<int64_t>(cu / blocks - 1024, blk);
    return lds > 0 ? (size_t)lds : 0;
#else
    (void)hidden;
    (void)slots;
    return 0;
#endif
}

template <Layout L, bool W_BF16, Epilogue EPI, int KC>
hipError_t launch_shape(const FinalizeArgs &a, hipStream_t s)
{
    if (a.top_k < 1 || a.top_k > kMaxTopK || (KC > 0 && a.top_k != KC) ||
        (KC < 0 && a.top_k > -KC))
        return hipErrorInvalidValue;
    const int n = a.hidden / 256;
    const int nv = 32 * n;
    const dim3 grid((unsigned)a.num_tokens);
    const int vpt = pick_vpt(L, n, KC);
    // Slots actually in flight: with top-k read at run time the batch may be
    // larger than top-k, and the cap must follow the rows really fetched.
    const int slots = std::min(KC > 0 ? KC : a.top_k, slots_in_flight(L, KC, vpt > 0 ? vpt : 1));
    const size_t lds = residency_lds(a.hidden, slots);
    switch (vpt) {
    case 8:
        if constexpr (vpt_reachable(8) || KC < 0)
            hipLaunchKernelGGL((finalize_kernel<L, W_BF16, EPI, KC, 8, true>), grid,
                               dim3(nv / 8), lds, s, a);
        break;
    case 4:
        if constexpr (vpt_reachable(4) || KC < 0)
            hipLaunchKernelGGL((finalize_kernel<L, W_BF16, EPI, KC, 4, true>), grid,
                               dim3(nv / 4), lds, s, a);
        break;
    case 2:
        if constexpr (vpt_reachable(2) || KC < 0)
            hipLaunchKernelGGL((finalize_kernel<L, W_BF16, EPI, KC, 2, true>), grid,
                               dim3(nv / 2), lds, s, a);
        break;
    case 1:
        if constexpr (vpt_reachable(1) || KC < 0)
            hipLaunchKernelGGL((finalize_kernel<L, W_BF16, EPI, KC, 1, true>), grid,
                               dim3(nv), lds, s, a);
        break;
    default:   // n odd: 32 (n + 1) threads, the last half wave idle
        hipLaunchKernelGGL((finalize_kernel<L, W_BF16, EPI, KC, 1, false>), grid,
                           dim3(nv + 32), lds, s, a);
        break;
    }
    return hipGetLastError();
}

// Compile-time slot counts for the common top-k values; other top-k read at
// run time, by a kernel sized for 8 slots up to 8, in batches beyond.
template <Layout L, bool W_BF16, Epilogue EPI>
hipError_t launch_topk(const FinalizeArgs &a, hipStream_t s)
{
    switch (a.top_k) {
    case 8:
        return launch_shape<L, W_BF16, EPI, 8>(a, s);
    case 16:
        return launch_shape<L, W_BF16, EPI, 16>(a, s);
    default:
        if (a.top_k <= 2)
            return launch_shape<L, W_BF16, EPI, small_topk_kc(2)>(a, s);
        if (a.top_k <= 4)
            return launch_shape<L, W_BF16, EPI, small_topk_kc(4)>(a, s);
        return a.top_k < 8 ? launch_shape<L, W_BF16, EPI, small_topk_kc(7)>(a, s)
                           : launch_shape<L, W_BF16, EPI, 0>(a, s);
    }
}

template <Epilogue EPI>
hipError_t launch_index_map(const FinalizeArgs &a, hipStream_t s)
{
    return a.weights_bf16 ? launch_topk<Layout::kIndexMap, true, EPI>(a, s)
                          : launch_topk<Layout::kIndexMap, false, EPI>(a, s);
}

}  // namespace

hipError_t launch_finalize(const FinalizeArgs &a, Layout layout, Epilogue epi, hipStream_t s)
{
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
            return launch_shape<Layout::kDirect, false, Epilogue::kRmsNorm, 1>(a, s);
        case Epilogue::kRmsNormWeightFirst:
            return launch_shape<Layout::kDirect, false, Epilogue::kRmsNormWeightFirst, 1>(a, s);
        case Epilogue::kResidualNorm:
            return launch_shape<Layout::kDirect, false, Epilogue::kResidualNorm, 1>(a, s);
        default:
            break;
        }
        break;
    }
    return hipErrorInvalidValue;
}

}  // namespace mf
