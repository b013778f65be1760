// A recording stand-in for mf::launch_finalize, linked with the C ABI's host
// code (moe_expert_output_finalize_amd/csrc/capi.cpp) into builds that run
// on the CPU only: the host-validation tests load one of them through ctypes,
// and the sanitizer test links another, built with AddressSanitizer and
// UndefinedBehaviorSanitizer, into tests/capi_sanitize_driver.c.
//
// Nothing here touches a GPU.  A "launch" is planned as the real launcher
// plans it (plan.hpp): the kernel variant and team for the call's shape, and
// the split of its tokens into launches of at most 2^31 work-items.  The
// stand-in checks what the C ABI handed over (pointers present and aligned
// where the kernels dereference them, sizes consistent, every token covered
// by exactly one launch whose work-item count fits the limit) and records
// the result for the tests to read back.
#include <stdint.h>
#include <string.h>

#include "args.hpp"
#include "plan.hpp"

namespace {

struct Record {
    int calls;           // launch_finalize calls since the last reset
    int layout, epi;     // of the last call
    int64_t num_tokens;
    int hidden, top_k;
    int kc, vpt, team, tpw;
    int64_t launches;    // kernel launches the last call was split into
    int64_t max_tokens;  // tokens per launch at most
    int64_t blocks;      // workgroups per CU the launcher reserves LDS for, 256 CUs
    int violations;      // contract violations seen since the last reset
    int fail_next;       // error code the next call returns (0: none)
};

Record g_rec;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

namespace mf {

int launch_finalize(const FinalizeArgs &a, Layout layout, Epilogue epi, void *stream)
{
    (void)stream;
    Record &r = g_rec;
    r.calls += 1;
    r.layout = static_cast<int>(layout);
    r.epi = static_cast<int>(epi);
    r.num_tokens = a.num_tokens;
    r.hidden = a.hidden;
    r.top_k = a.top_k;
    if (r.fail_next) {
        const int code = r.fail_next;
        r.fail_next = 0;
        return code;
    }
    // What the kernels dereference must be there.
    const bool idx_map = layout == Layout::kIndexMap;
    const bool direct = layout == Layout::kDirect;
    if (a.num_tokens <= 0 || a.hidden < 256 || a.hidden > 8192 || a.hidden % 256 != 0 ||
        a.top_k < 1 || a.top_k > kMaxTopK || a.token_base != 0)
        r.violations += 1;
    if (!a.out || !aligned16(a.out) || (!a.rows && !(idx_map && a.num_rows == 0)) ||
        (a.rows && !aligned16(a.rows)))
        r.violations += 1;
    if (!direct && !a.weights)
        r.violations += 1;
    if (idx_map && (!a.idx || a.row_stride < a.hidden || a.row_stride % 8 != 0))
        r.violations += 1;
    if (epi == Epilogue::kRmsNorm || epi == Epilogue::kRmsNormWeightFirst)
        if (!a.gain || !aligned16(a.gain))
            r.violations += 1;
    if (epi == Epilogue::kResidualNorm &&
        (!a.residual || !aligned16(a.residual) || (a.has_next && !a.out2)))
        r.violations += 1;
    if (epi == Epilogue::kRound && !idx_map)
        r.violations += 1;
    // Plan as the launcher does and walk the launches.
    const LaunchPlan p = plan_launch(idx_map, direct, a.hidden, direct ? 1 : a.top_k);
    r.kc = p.kc;
    r.vpt = p.vpt;
    r.team = p.team;
    r.tpw = p.tpw;
    r.max_tokens = p.max_tokens;
    r.blocks = residency_blocks(idx_map, a.hidden * p.tpw, p.slots,
                                (a.num_tokens + p.tpw - 1) / p.tpw, 256);
    r.launches = 0;
    int64_t covered = 0;
    for (int64_t t0 = 0; t0 < a.num_tokens; t0 += p.max_tokens) {
        const int64_t n = a.num_tokens - t0 < p.max_tokens ? a.num_tokens - t0 : p.max_tokens;
        if (n <= 0 || (n + p.tpw - 1) / p.tpw * p.team > kMaxThreadsPerLaunch || t0 != covered ||
            (n < p.max_tokens ? false : n % p.tpw != 0))
            r.violations += 1;
        covered += n;
        r.launches += 1;
    }
    if (covered != a.num_tokens || p.team % kWave != 0 || p.team > max_team(p.vpt ? p.vpt : 1))
        r.violations += 1;
    return 0;
}

const char *launch_error_string(int code)
{
    return code == 0 ? "no error" : "launch refused by the host test stand-in";
}

}  // namespace mf

extern "C" {

// Forget every recorded call.
void mf_test_reset(void) { memset(&g_rec, 0, sizeof g_rec); }

// Make the next launch fail with `code` (non-zero).
void mf_test_fail_next_launch(int code) { g_rec.fail_next = code; }

// The record, as 14 int64 values: calls, layout, epilogue, num_tokens, hidden,
// top_k, kc, vpt, team, tpw, launches, max_tokens, blocks, violations.
void mf_test_record(int64_t *out)
{
    const Record &r = g_rec;
    const int64_t v[14] = {r.calls,    r.layout,   r.epi,        r.num_tokens, r.hidden,
                           r.top_k,    r.kc,       r.vpt,        r.team,       r.tpw,
                           r.launches, r.max_tokens, r.blocks,   r.violations};
    memcpy(out, v, sizeof v);
}

// Token block of workgroup b in an n-workgroup grid of a multi-token-wave
// kernel, with the library's own run length (the map the kernels use).
unsigned mf_test_xcd_run_block(unsigned b, unsigned n)
{
    return mf::xcd_run_block(b, n, MF_XCD_RUN);
}

}  // extern "C"
