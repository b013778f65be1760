// Launch planning shared by the gfx950 kernels (as compile-time constants)
// and the host launcher (finalize_kernels.hip): team shape, slots in flight,
// residency and the split of a call into launches.  Plain C++ with no HIP
// types, so host tests can check the arithmetic on the CPU.
#pragma once

#include <stdint.h>

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
// Slots an index-map workgroup keeps in flight, by vectors per thread (one,
// two): a token with more slots streams them through a rolling window of
// this many.  Token-major tokens with more slots than fit arrive in batches
// instead: a token's rows are one contiguous block, fetched fastest in
// bursts (a rolling window measured 4 % slower at top-k 16 and hidden 2048,
// and no faster at any other shape).
#ifndef MF_ROLL_WINDOW_VPT1
#define MF_ROLL_WINDOW_VPT1 16
#endif
#ifndef MF_ROLL_WINDOW_VPT2
#define MF_ROLL_WINDOW_VPT2 8
#endif
// Hidden 256 is 32 vectors, half of a 64-lane wave: at small top-k
// several tokens share each one-wave workgroup, as many (2, 4 or 8) as keep
// tokens x slots at most this (0: one token per workgroup with half the
// wave idle).
#ifndef MF_WAVE_TOKEN_SLOTS
#define MF_WAVE_TOKEN_SLOTS 4
#endif
// Hidden 512 (64 vectors, a whole wave) at top-k 1: two tokens per wave,
// 32 lanes of two vectors each (0: one token per wave).
#ifndef MF_WAVE_TOKENS_512
#define MF_WAVE_TOKENS_512 1
#endif
#ifndef MF_INFLIGHT_KB_PER_CU
#define MF_INFLIGHT_KB_PER_CU 128 // > 0: cap resident workgroups so that their row
                                  // loads in flight total about this much per CU
#endif
// An index-map call whose tokens fit on the device at up to this many
// workgroups per CU runs them all in one round instead (0: off).
#ifndef MF_ONE_ROUND_MAX_BLOCKS
#define MF_ONE_ROUND_MAX_BLOCKS 8
#endif
// Multi-token waves (hidden 256) hand runs of this many consecutive
// workgroups to one XCD, so that a cache line of slot metadata is fetched
// into one XCD's L2 rather than every XCD's (0 or 1: workgroup b finalizes
// token block b).
#ifndef MF_XCD_RUN
#define MF_XCD_RUN 32
#endif

namespace mf {

constexpr int kWave = 64;
// XCDs of an MI355X; the dispatcher deals workgroup b of a grid to XCD b % 8.
constexpr unsigned kXcds = 8;
constexpr int kMaxTopK = 32;   // the entry points reject larger top-k
constexpr int kMaxWaves = 16;
// Work-items one launch may span.  The dispatch packet counts the grid in
// 32-bit work-items; a call whose tokens need more is split into launches of
// at most this many (2^31, which also keeps every runtime-side product of
// grid and team inside a signed 32-bit integer).
constexpr int64_t kMaxThreadsPerLaunch = int64_t(1) << 31;

inline constexpr int layout_max_vecs(bool index_map)
{
    return index_map ? MF_MAX_VECS_INDEX_MAP : MF_MAX_VECS_TOKEN_MAJOR;
}

// Row vectors one thread keeps in flight.  One vector per thread means teams
// of up to 1024 threads, whose launch bound leaves 128 VGPRs per thread: at
// most 16 vectors (64 VGPRs) there.
constexpr int max_vecs(bool index_map, int vpt)
{
    return vpt == 1 && layout_max_vecs(index_map) > 16 ? 16 : layout_max_vecs(index_map);
}

// Slot-count template argument:
//   KC > 0   top-k is KC (8 and 16);
//   KC < 0   top-k is read at run time and is at most -KC; registers are
//            sized for -KC slots, so a small top-k keeps a small register
//            footprint and high occupancy, and a larger one wastes at most a
//            few slots (-2, -4, -8, -12, -16, -24, -32).
constexpr int small_topk_kc(int top_k) { return top_k <= 2 ? -2 : top_k <= 4 ? -4 : -8; }

// The KC a top-k is served by.
constexpr int kc_for_topk(int top_k)
{
    return top_k == 8 ? 8 : top_k == 16 ? 16 : top_k < 8 ? small_topk_kc(top_k)
         : top_k <= 12 ? -12 : top_k <= 16 ? -16 : top_k <= 24 ? -24 : -32;
}

// The index-map window for `vpt` vectors per thread.
constexpr int window(int vpt)
{
    return vpt == 1 ? MF_ROLL_WINDOW_VPT1 : vpt == 2 ? MF_ROLL_WINDOW_VPT2 : MF_MAX_VECS_INDEX_MAP / vpt;
}

// Whether a token's slots stream through a rolling window (index map, more
// slots than the window) instead of arriving in one batch or several.
constexpr bool rolling(bool index_map, int kc, int vpt)
{
    return index_map && (kc < 0 ? -kc : kc) > window(vpt);
}

// Slots whose rows one workgroup has in flight at once: all of a token's
// when they fit (the window on the index map, max_vecs on token-major
// rows), else the window, else batches of max_vecs / VPT slots.
constexpr int slots_in_flight(bool index_map, int kc, int vpt)
{
    const int want = kc < 0 ? -kc : kc;
    if (index_map)
        return want <= window(vpt) ? want : window(vpt);
    return want * vpt <= max_vecs(false, vpt) ? want : max_vecs(false, vpt) / vpt;
}

constexpr int max_team(int vpt) { return vpt == 1 ? 1024 : vpt == 2 ? 512 : 256; }

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
constexpr bool team_fits(int n, int vpt)
{
    return (32 * n) % vpt == 0 && (32 * n / vpt) % kWave == 0 && 32 * n / vpt >= kWave &&
           32 * n / vpt <= max_team(vpt);
}

// Vectors per thread for hidden = 256 n: one for index-map rows up to
// MF_INDEX_MAP_VPT1_MAX_HIDDEN, else the first of MF_VPT_ORDER whose team
// fits; 0 if none (then one vector per thread with the last half wave idle).
// On the index map, a run-time top-k below 8 (kc < 0) widens that by
// 8 / -kc where the team still fits, so a thread keeps about as many row
// vectors in flight as at top-k 8 while workgroups stay small enough for
// high occupancy (2-8 % faster at top-k 2 and 4; token-major rows measured
// faster without it).
constexpr int pick_vpt(bool index_map, int n, int kc)
{
    int base = 0;
    if (index_map && 256 * n <= MF_INDEX_MAP_VPT1_MAX_HIDDEN && n % 2 == 0 && vpt_reachable(1)) {
        base = 1;
    } else {
        constexpr int order[] = {MF_VPT_ORDER};
        for (int vpt : order)
            if (team_fits(n, vpt)) {
                base = vpt;
                break;
            }
    }
    if (index_map && kc < 0 && base > 0)
        for (int vpt = (base * 8 / -kc < 8 ? base * 8 / -kc : 8); vpt > base; vpt /= 2)
            if (team_fits(n, vpt))
                return vpt;
    return base;
}

// Whether pick_vpt returns `vpt` for some hidden size of the envelope
// (256 n, n = 1..32): kernels for other values are not instantiated.
constexpr bool vpt_possible(bool index_map, int kc, int vpt)
{
    for (int n = 1; n <= 32; ++n)
        if (pick_vpt(index_map, n, kc) == vpt)
            return true;
    return false;
}

// The token block workgroup b of an n-workgroup grid finalizes when runs of
// `run` consecutive blocks go to one XCD: XCD x = b % kXcds receives its
// i-th workgroup (i = b / kXcds) from run i / run, and runs are interleaved
// over the XCDs in block order.  The grid's last partial group of
// kXcds * run workgroups keeps b, so the map is a bijection on [0, n) for
// any n (and any XCD count: only the locality depends on it).
constexpr unsigned xcd_run_block(unsigned b, unsigned n, unsigned run)
{
    const unsigned span = kXcds * run;
    if (run <= 1 || b >= n / span * span)
        return b;
    const unsigned x = b % kXcds, i = b / kXcds;
    return (i / run * kXcds + x) * run + i % run;
}

// Tokens a one-wave workgroup of kernels for slot-count argument kc
// finalizes at hidden 256: a token of 32 vectors and at most 4 slots moves
// 0.5-2 KiB, and one such token per wave leaves the CU's 32 waves bound by
// latency.  The largest of 8, 4, 2 with tokens x slots within
// MF_WAVE_TOKEN_SLOTS (at least 2), for kc up to 4 slots and for the
// run-time kernel of up to 8 (top-k 5-7, where one token per wave leaves
// half of it idle: index map 3-4 % faster with two); else 1 (the
// compile-time 8 was 1.3 % slower with two, and above 8 slots every slot in
// flight at once loses to the rolling window).
constexpr int wave_tokens(int kc)
{
    const int k = kc < 0 ? -kc : kc;
    if (MF_WAVE_TOKEN_SLOTS <= 0 || (k > 4 && kc != -8))
        return 1;
    int t = 8;
    while (t > 2 && t * k > MF_WAVE_TOKEN_SLOTS)
        t /= 2;
    return t;
}

// Tokens one workgroup finalizes: wave_tokens(kc) at hidden 256, two at
// hidden 512 with one slot (a token's single row is 1 KiB, and one token per
// wave leaves too few bytes in flight behind the index round trip), else one.
constexpr int tokens_per_workgroup(int hidden, int kc)
{
    return hidden == 256                           ? wave_tokens(kc)
           : hidden == 512 && kc == 1 && MF_WAVE_TOKENS_512 ? 2
                                                   : 1;
}

// How one call is launched.
struct LaunchPlan {
    int kc;               // slot-count template argument
    int vpt;              // 16-byte vectors per thread (0: one, last half wave idle)
    int team;             // threads per workgroup
    int tpw;              // tokens per workgroup (2, 4 or 8: one wave at hidden 256)
    int slots;            // slots per token whose rows a workgroup has in flight at once
    bool exact;           // hidden / 8 == team * vpt (per token)
    int64_t max_tokens;   // tokens per launch at most (a multiple of tpw)
};

constexpr LaunchPlan plan_launch(bool index_map, bool direct, int hidden, int top_k)
{
    LaunchPlan p{};
    const int n = hidden / 256;
    p.kc = direct ? 1 : kc_for_topk(top_k);
    // Top-k 1 at hidden 256 runs slot count 1 when that packs more tokens
    // per wave than the run-time kernel for 1-2 slots; at hidden 512 slot
    // count 1 holds two tokens per wave.
    if (top_k == 1 && ((hidden == 256 && wave_tokens(1) > wave_tokens(p.kc)) ||
                       (hidden == 512 && MF_WAVE_TOKENS_512)))
        p.kc = 1;
    p.tpw = tokens_per_workgroup(hidden, p.kc);
    const int kk = p.kc > 0 ? p.kc : top_k;
    if (p.tpw > 1) {   // one wave, 64 / tpw lanes per token, all slots at once
        p.vpt = 32 * n * p.tpw / kWave;
        p.exact = true;
        p.team = kWave;
        p.slots = kk;
    } else {
        p.vpt = pick_vpt(index_map, n, p.kc);
        p.exact = p.vpt > 0;
        p.team = p.vpt > 0 ? 32 * n / p.vpt : 32 * n + 32;
        const int win = slots_in_flight(index_map, p.kc, p.vpt > 0 ? p.vpt : 1);
        p.slots = kk < win ? kk : win;
    }
    p.max_tokens = kMaxThreadsPerLaunch / p.team * p.tpw;
    return p;
}

// Workgroups a CU should hold, 0 for no cap.  Normally
// ceil(MF_INFLIGHT_KB_PER_CU / in-flight bytes per workgroup), clamped to
// 2..32: beyond that, extra concurrent gathers do not raise bandwidth; they
// stretch every token's lifetime and with it the tail of the launch
// (measured: 2-5 % faster on every large workload than residency limited by
// registers).  The upper end is the 32 waves a CU holds: small rows run one-
// wave workgroups, and a clamp at 16 left them half the bytes in flight
// (hidden 256: 13-27 % slower, hidden 512 / top-k 2: 13 %).  But an
// index-map call with more tokens than that holds on
// the device's `cus` CUs, yet no more than MF_ONE_ROUND_MAX_BLOCKS per CU,
// gets ceil(tokens / cus): all of its tokens start at once, with no second
// round whose last workgroups run on a nearly idle device.  Registers may
// still hold fewer, and the raised cap then still shortens the rounds.
// Measured for 585-2048 tokens: 1-3 % faster at hidden 4096 / top-k 8, 4-10 %
// at hidden 2048 / top-k 16, up to 7 % at hidden 2048 / top-k 32 (768
// tokens); within 1.4 % either way at hidden 4096 / top-k 16, whose cap
// already holds more than the target in flight; at hidden 4096 / top-k 4,
// 5 % faster at 1170 tokens and 2 % slower at 1560.  Raising it only where
// the kernel's occupancy confirms a single round gave up most of the gains;
// token-major rows gained nothing consistent.
constexpr int64_t residency_blocks(bool index_map, int hidden, int slots, int64_t tokens,
                                   int cus)
{
    if (MF_INFLIGHT_KB_PER_CU <= 0 || hidden <= 0 || slots <= 0)
        return 0;
    const int64_t per_block = 2LL * hidden * slots;   // row bytes in flight
    const int64_t want = ((int64_t)MF_INFLIGHT_KB_PER_CU * 1024 + per_block - 1) / per_block;
    // A workgroup with at most 8 KiB of rows in flight spends much of its
    // life in its fixed phases (the index round trip, the reduction, the
    // stores), so it gets the full 32 (hidden 256 at top-k 12 and 16: 7-11 %
    // faster than 22 and 16 per CU; no change elsewhere).
    const int64_t blocks = per_block <= 8 * 1024 ? 32 : want < 2 ? 2 : want > 32 ? 32 : want;
    if (index_map && cus > 0 && tokens > blocks * cus) {
        const int64_t need = (tokens + cus - 1) / cus;
        if (need <= MF_ONE_ROUND_MAX_BLOCKS)
            return need;
    }
    return blocks;
}

// Dynamic LDS to reserve per workgroup so that a CU holds `blocks`
// workgroups (residency_blocks), given the device's LDS per CU and per
// workgroup and the kernel's own static LDS.  0 when no cap applies.
constexpr int64_t residency_lds(int64_t blocks, int64_t lds_per_cu, int64_t lds_per_block,
                                int64_t static_lds)
{
    if (blocks <= 0 || lds_per_cu <= 0 || lds_per_block <= 0)
        return 0;
    // Leave 1 KiB of the CU's share unclaimed, and never ask for more than a
    // workgroup may hold besides the kernel's own LDS.
    int64_t lds = lds_per_cu / blocks - 1024;
    if (lds > lds_per_block - static_lds)
        lds = lds_per_block - static_lds;
    return lds > 0 ? lds : 0;
}

}  // namespace mf
