"""Host-side tests of the C ABI (no GPU needed).

The library must load and export every function include/moe_finalize.h
declares, with the binding's prototypes matching the header.  Argument
validation, the launch plan and the split of large token counts into
launches run against the host-check build of the same C ABI code, whose
launcher is a recording stand-in: nothing here can reach a GPU.
"""
import ctypes
import os
import re

import pytest

import capi_cases as cc
import moe_expert_output_finalize_amd as mf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_finalize.h")
HOSTCHECK = os.path.join(ROOT, "tests", "libmf_hostcheck.so")


def declared_functions():
    src = open(HEADER).read()
    return re.findall(r"MF_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)


def test_header_declares_the_entry_points():
    names = set(declared_functions())
    assert {"moe_finalize_rmsnorm", "moe_finalize", "beam_moe_finalize", "mf_rmsnorm",
            "beam_moe_finalize_norm_residual_norm", "beam_norm_residual_norm",
            "mf_status_string", "mf_last_error_message"} <= names


def test_library_exports_every_declared_symbol():
    so = ctypes.CDLL(mf.LIB_PATH)
    for name in declared_functions():
        assert hasattr(so, name), f"{name} declared in the header but not exported"


def declared_prototypes():
    """name -> list of parameter declarations, from the header's MF_API lines."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    protos = {}
    for m in re.finditer(r"MF_API\s+[\w\s\*]+?\b(\w+)\s*\(([^;]*?)\)\s*;", src, flags=re.S):
        params = [p.strip() for p in m.group(2).split(",") if p.strip()]
        protos[m.group(1)] = [] if params == ["void"] else params
    return protos


_CTYPE = {"int64_t": ctypes.c_int64, "int32_t": ctypes.c_int32, "float": ctypes.c_float,
          "int": ctypes.c_int}


def test_binding_argtypes_match_the_header():
    """The Python binding declares every entry point with the header's
    parameter count and, for scalars, the header's C type (pointers are
    passed as void *)."""
    protos = declared_prototypes()
    assert len(protos) == len(declared_functions())
    for name, params in protos.items():
        argtypes = getattr(mf.lib, name).argtypes
        assert argtypes is not None and len(argtypes) == len(params), name
        for decl, ct in zip(params, argtypes):
            if "*" in decl:
                assert ct in (ctypes.c_void_p, ctypes.c_char_p), (name, decl)
            else:
                ctype = decl.replace("const", "").split()[0]
                assert ct is _CTYPE[ctype], (name, decl, ct)


def test_status_strings():
    for code in range(7):
        s = mf.lib.mf_status_string(code).decode()
        assert s and s != "unknown status"
    assert mf.lib.mf_status_string(99).decode() == "unknown status"
    assert mf.lib.mf_last_error_message().decode() == ""


# ------------------------------------------- validation (no GPU involved) ---
#
# The cases run against tests/libmf_hostcheck.so: the same C ABI host code
# (csrc/capi.cpp) as the real library, linked with a recording stand-in for
# the launcher instead of the HIP kernels, so a case that validation wrongly
# accepts is recorded, never launched.

@pytest.fixture(scope="module")
def host():
    if not os.path.exists(HOSTCHECK):
        pytest.fail(f"{HOSTCHECK} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(HOSTCHECK)
    cc.declare(lib)
    lib.mf_test_record.argtypes = [ctypes.POINTER(ctypes.c_int64)]
    lib.mf_test_fail_next_launch.argtypes = [ctypes.c_int]
    lib.mf_last_error_message.restype = ctypes.c_char_p
    return lib


def record(lib) -> dict:
    buf = (ctypes.c_int64 * 14)()
    lib.mf_test_record(buf)
    keys = ("calls", "layout", "epi", "num_tokens", "hidden", "top_k", "kc", "vpt", "team",
            "tpw", "launches", "max_tokens", "blocks", "violations")
    return dict(zip(keys, list(buf)))


@pytest.mark.parametrize("case", cc.CASES, ids=cc.case_id)
def test_validation(host, case):
    """Each invalid argument is rejected with its status and launches
    nothing; each valid call launches exactly once with arguments the
    kernels can use, and zero-row calls launch nothing."""
    fn, over, want = case
    host.mf_test_reset()
    assert cc.ctypes_call(host, fn, over) == want
    rec = record(host)
    zero_rows = any(over.get(k) == 0 for k in ("T", "live"))
    assert rec["calls"] == (1 if want == cc.OK and not zero_rows else 0)
    assert rec["violations"] == 0


@pytest.mark.parametrize("case", cc.SPLIT_CASES, ids=cc.case_id)
def test_token_counts_beyond_one_launch_are_split(host, case):
    """Calls whose grid would pass 2^31 work-items are split into launches
    that each fit, cover every token once and keep the call's plan."""
    fn, over, launches = case
    host.mf_test_reset()
    assert cc.ctypes_call(host, fn, over) == cc.OK
    rec = record(host)
    assert rec["calls"] == 1 and rec["violations"] == 0
    assert rec["launches"] == launches
    assert rec["max_tokens"] // rec["tpw"] * rec["team"] <= 2 ** 31
    assert (rec["launches"] - 1) * rec["max_tokens"] < rec["num_tokens"]
    assert rec["launches"] * rec["max_tokens"] >= rec["num_tokens"]


def test_largest_token_count_at_every_hidden_size(host):
    """INT32_MAX tokens at every hidden size of the envelope and several top-k
    on both layouts: accepted, and split into launches within the limit."""
    for H in range(256, 8193, 256):
        for K in (1, 5, 8, 13, 16, 32):
            for fn, over in (("moe_finalize", dict(H=H, stride=H, K=K, T=cc.INT32_MAX)),
                             ("beam_moe_finalize", dict(H=H, K=K, cap=cc.INT32_MAX,
                                                        wrows=cc.INT32_MAX,
                                                        live=cc.INT32_MAX))):
                host.mf_test_reset()
                assert cc.ctypes_call(host, fn, over) == cc.OK, (fn, H, K)
                rec = record(host)
                assert rec["violations"] == 0 and rec["calls"] == 1, (fn, H, K, rec)
                assert rec["max_tokens"] // rec["tpw"] * rec["team"] <= 2 ** 31


@pytest.mark.parametrize("fn,over,kc,vpt,team,tpw", [
    ("moe_finalize_rmsnorm", dict(), 8, 1, 512, 1),
    ("moe_finalize_rmsnorm", dict(H=7168, stride=7168, K=32), -32, 2, 448, 1),
    ("moe_finalize_rmsnorm", dict(H=2048, stride=2048, K=12), -12, 1, 256, 1),
    ("moe_finalize_rmsnorm", dict(H=4096, K=2), -2, 4, 128, 1),
    ("moe_finalize", dict(H=256, stride=256, K=1), 1, 2, 64, 4),       # four tokens per wave
    ("moe_finalize", dict(H=256, stride=256, K=2), -2, 1, 64, 2),      # two tokens per wave
    ("moe_finalize", dict(H=512, stride=512, K=1), 1, 2, 64, 2),       # two tokens of 64 vectors
    ("moe_finalize", dict(H=512, stride=512, K=2), -2, 1, 64, 1),      # one token per wave
    ("beam_moe_finalize", dict(H=512, K=1), 1, 2, 64, 2),
    ("mf_rmsnorm", dict(H=512, stride=512), 1, 2, 64, 2),
    ("moe_finalize", dict(H=768, stride=768, K=1), -2, 0, 128, 1),     # last half wave idle
    ("beam_moe_finalize", dict(), 8, 2, 448, 1),
    ("beam_moe_finalize", dict(K=17), -24, 2, 448, 1),
    ("beam_moe_finalize", dict(H=256, K=3), -4, 1, 64, 2),
    ("beam_moe_finalize", dict(H=256, K=1), 1, 2, 64, 4),
    ("beam_moe_finalize", dict(H=256, K=6), -8, 1, 64, 2),       # run-time 8 slots: two
    ("beam_moe_finalize", dict(H=256, K=8), 8, 0, 64, 1),        # compile-time 8: one token
    ("moe_finalize", dict(H=256, stride=256, K=12), -12, 0, 64, 1),
    ("mf_rmsnorm", dict(), 1, 2, 256, 1),
    ("mf_rmsnorm", dict(H=256, stride=256), 1, 2, 64, 4),
])
def test_launch_plan(host, fn, over, kc, vpt, team, tpw):
    """The kernel variant, team and tokens per workgroup the launcher picks
    for a few shapes."""
    host.mf_test_reset()
    assert cc.ctypes_call(host, fn, over) == cc.OK
    rec = record(host)
    assert (rec["kc"], rec["vpt"], rec["team"], rec["tpw"]) == (kc, vpt, team, tpw), rec


# Workgroups per CU the launcher reserves LDS for on a 256-CU device: about
# 128 KiB of rows in flight per CU (2..32 workgroups, 32 being the waves a
# CU holds; 32 outright for workgroups with at most 8 KiB of rows in
# flight), or, for an index-map call that fits at up to 8 per CU, all of its
# tokens at once: ceil(tokens / 256).
@pytest.mark.parametrize("fn,over,blocks", [
    ("moe_finalize_rmsnorm", dict(T=8192), 2),                      # 8 x 8 KiB rows: cap 2
    ("moe_finalize_rmsnorm", dict(T=512), 2),                       # one round already
    ("moe_finalize_rmsnorm", dict(T=513), 3),
    ("moe_finalize_rmsnorm", dict(T=585), 3),
    ("moe_finalize_rmsnorm", dict(T=2048), 8),
    ("moe_finalize_rmsnorm", dict(T=2049), 2),                      # would need 9 per CU
    ("moe_finalize", dict(H=2048, stride=2048, K=16, T=1170), 5),   # 16 x 4 KiB: cap 2
    ("moe_finalize", dict(H=4096, K=2, T=4096), 8),                 # 2 x 8 KiB: cap 8
    ("moe_finalize", dict(H=256, stride=256, K=1, T=8192), 32),     # tiny rows: cap 32
    ("beam_moe_finalize", dict(cap=1024, wrows=1024, live=585), 2), # token major: cap only
    ("mf_rmsnorm", dict(T=585), 32),                                # one 8 KiB row: 32
    ("moe_finalize", dict(H=256, stride=256, K=12, T=4096), 32),    # 12 x 512 B rows
    ("moe_finalize", dict(H=512, stride=512, K=10, T=4096), 13),    # 10 x 1 KiB rows
    ("mf_rmsnorm", dict(H=2048, stride=2048, T=585), 32),           # one 4 KiB row: 32
    ("moe_finalize", dict(H=512, stride=512, K=2, T=4096), 32),     # 2 x 1 KiB rows
])
def test_residency(host, fn, over, blocks):
    host.mf_test_reset()
    assert cc.ctypes_call(host, fn, over) == cc.OK
    rec = record(host)
    assert rec["violations"] == 0 and rec["blocks"] == blocks, rec


def test_failed_launch_is_reported(host):
    """A launch error becomes MF_ERR_LAUNCH_FAILED with a message, which the
    next successful call clears."""
    host.mf_test_reset()
    host.mf_test_fail_next_launch(98)
    assert cc.ctypes_call(host, "moe_finalize", {}) == cc.LAUNCH
    assert host.mf_last_error_message().decode().startswith("kernel launch failed")
    assert cc.ctypes_call(host, "moe_finalize", {}) == cc.OK
    assert host.mf_last_error_message().decode() == ""


def test_binding_rejects_host_tensors():
    import torch
    g = torch.zeros(8, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mf.moe_finalize(g, torch.zeros(1, 8), torch.zeros(1, 8, dtype=torch.int32),
                        torch.zeros(1, 256, dtype=torch.bfloat16))


@pytest.mark.parametrize("strategy", ["oneshot", "twoshot", "FUSED", ""])
def test_unknown_strategy_is_rejected(strategy):
    """The fused residual entry point takes the page's strategy keyword: None,
    "fused" or "unfused"; any other value raises ValueError before a tensor
    is looked at (so host tensors suffice here)."""
    import torch
    e = torch.zeros(1, 1, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="strategy"):
        mf.beam_moe_finalize_norm_residual_norm(e, torch.zeros(1, 1),
                                                torch.zeros(1, 256, dtype=torch.bfloat16),
                                                None, None, None, None, None, strategy=strategy)


def test_c_driver_links_against_the_library():
    """The plain-C driver of the GPU tests resolves libmoe_finalize.so and the
    HIP runtime; without arguments it prints its usage before any HIP call."""
    import subprocess
    driver = os.path.join(ROOT, "tests", "capi_c_driver")
    assert os.path.exists(driver), "run __graft_entry__.build() first"
    r = subprocess.run([driver], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage:" in r.stderr


@pytest.mark.parametrize("n", [1, 7, 63, 255, 256, 257, 1000, 4096 + 17, 32768])
def test_xcd_runs_are_a_permutation_of_token_blocks(host, n):
    """Multi-token-wave kernels hand runs of consecutive token blocks to one
    XCD (workgroup b runs on XCD b % 8): every block of the grid is still
    finalized exactly once, and in the full groups XCD x's successive
    workgroups take consecutive blocks."""
    host.mf_test_xcd_run_block.argtypes = [ctypes.c_uint, ctypes.c_uint]
    host.mf_test_xcd_run_block.restype = ctypes.c_uint
    m = [host.mf_test_xcd_run_block(b, n) for b in range(n)]
    assert sorted(m) == list(range(n))
    run = 32
    full = n // (8 * run) * (8 * run)
    for b in range(full - 8):
        if (b // 8) % run != run - 1:
            assert m[b + 8] == m[b] + 1, (b, m[b], m[b + 8])
    assert m[full:] == list(range(full, n))

