"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/moe_finalize.h
declares, and reject bad arguments with the documented status before any HIP
call.  Zero-row calls return MF_OK without launching.  The pointers used
here are never dereferenced: every call below fails validation or has
nothing to do.
"""
import ctypes
import os
import re

import pytest

import moe_expert_output_finalize_amd as mf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_finalize.h")

OK, NULLP, SHAPE, DTYPE, ALIGN, ARG = 0, 1, 2, 3, 4, 5
BF16, FP32 = 1, 2
P = 0x10000          # a 16-byte aligned fake device address (never dereferenced)


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


def rmsnorm(**over):
    a = dict(g=P, rows=128, stride=4096, w=P, wdt=FP32, idx=P, nw=P, out=P, T=16, H=4096, K=8,
             eps=1e-6, gc=1.0, wbn=0, stream=None)
    a.update(over)
    return mf.lib.moe_finalize_rmsnorm(a["g"], a["rows"], a["stride"], a["w"], a["wdt"],
                                       a["idx"], a["nw"], a["out"], a["T"], a["H"], a["K"],
                                       a["eps"], a["gc"], a["wbn"], a["stream"])


def finalize(**over):
    a = dict(g=P, rows=128, stride=4096, w=P, wdt=FP32, idx=P, out=P, T=16, H=4096, K=8,
             stream=None)
    a.update(over)
    return mf.lib.moe_finalize(a["g"], a["rows"], a["stride"], a["w"], a["wdt"], a["idx"],
                               a["out"], a["T"], a["H"], a["K"], a["stream"])


def beam(**over):
    a = dict(e=P, cap=4096, K=8, H=7168, w=P, wrows=4096, out=P, live=3000, pw=None,
             scale=2.5, eps=0.0, norm=0, stream=None)
    a.update(over)
    return mf.lib.beam_moe_finalize(a["e"], a["cap"], a["K"], a["H"], a["w"], a["wrows"],
                                    a["out"], a["live"], a["pw"], a["scale"], a["eps"],
                                    a["norm"], a["stream"])


# Each case would be valid but for the one named change; T = 0 keeps the
# valid base from launching anything.
@pytest.mark.parametrize("over,want", [
    (dict(T=0), OK),
    (dict(T=0, g=None, w=None, idx=None, nw=None, out=None), OK),
    (dict(T=0, H=2048, K=4), OK), (dict(T=0, H=256, K=1), OK), (dict(T=0, H=8192, K=32, stride=8192), OK),
    (dict(H=2000), SHAPE), (dict(H=8448, stride=8448), SHAPE), (dict(K=0), SHAPE), (dict(K=33), SHAPE),
    (dict(T=-1), SHAPE), (dict(rows=-1), SHAPE),
    (dict(T=1 << 31), SHAPE), (dict(stride=4088), SHAPE),
    (dict(stride=4100), ALIGN), (dict(wdt=0), DTYPE), (dict(wdt=3), DTYPE),
    (dict(g=None), NULLP), (dict(w=None), NULLP), (dict(idx=None), NULLP),
    (dict(nw=None), NULLP), (dict(out=None), NULLP),
    (dict(g=P + 2), ALIGN), (dict(w=P + 4), ALIGN), (dict(idx=P + 8), ALIGN),
    (dict(nw=P + 2), ALIGN), (dict(out=P + 8), ALIGN),
])
def test_rmsnorm_validation(over, want):
    assert rmsnorm(**over) == want


@pytest.mark.parametrize("over,want", [
    (dict(T=0), OK), (dict(T=0, H=256, K=1), OK), (dict(T=0, H=8192, K=32, stride=8192), OK),
    (dict(T=0, rows=0, g=None), OK),
    (dict(H=128), SHAPE), (dict(H=8448, stride=8448), SHAPE), (dict(H=4000), SHAPE),
    (dict(K=0), SHAPE), (dict(K=33), SHAPE), (dict(stride=2048, H=4096), SHAPE),
    (dict(stride=4100), ALIGN), (dict(wdt=7), DTYPE),
    (dict(out=None), NULLP), (dict(g=None), NULLP), (dict(g=P + 4), ALIGN),
])
def test_finalize_validation(over, want):
    assert finalize(**over) == want


@pytest.mark.parametrize("over,want", [
    (dict(live=0), OK), (dict(live=0, e=None, w=None, out=None), OK),
    (dict(live=0, norm=1, pw=P, eps=1e-6), OK),
    (dict(K=0), SHAPE), (dict(K=33), SHAPE), (dict(H=7000), SHAPE), (dict(H=0), SHAPE),
    (dict(H=8448), SHAPE), (dict(live=4097), SHAPE), (dict(wrows=2999), SHAPE),
    (dict(cap=-1), SHAPE), (dict(live=-1), SHAPE),
    (dict(pw=P, norm=0), ARG), (dict(e=None), NULLP), (dict(w=None), NULLP),
    (dict(out=None), NULLP), (dict(e=P + 8), ALIGN), (dict(w=P + 2), ALIGN),
    (dict(out=P + 2), ALIGN), (dict(pw=P + 2, norm=1), ALIGN),
])
def test_beam_validation(over, want):
    assert beam(**over) == want


def norm(**over):
    a = dict(x=P, stride=4096, nw=P, out=P, T=16, H=4096, eps=1e-6, gc=1.0, wbn=0, stream=None)
    a.update(over)
    return mf.lib.mf_rmsnorm(a["x"], a["stride"], a["nw"], a["out"], a["T"], a["H"], a["eps"],
                             a["gc"], a["wbn"], a["stream"])


@pytest.mark.parametrize("over,want", [
    (dict(T=0), OK), (dict(T=0, x=None, nw=None, out=None), OK), (dict(T=0, H=256), OK),
    (dict(H=200), SHAPE), (dict(H=8448, stride=8448), SHAPE), (dict(T=-1), SHAPE),
    (dict(stride=4000), SHAPE), (dict(stride=4100), ALIGN),
    (dict(x=None), NULLP), (dict(nw=None), NULLP), (dict(out=None), NULLP),
    (dict(x=P + 2), ALIGN), (dict(nw=P + 8), ALIGN), (dict(out=P + 4), ALIGN),
])
def test_standalone_norm_validation(over, want):
    assert norm(**over) == want


def fused_rn(**over):
    a = dict(e=P, cap=16384, K=16, H=2048, w=P, wrows=16384, res=P, pw=P, nw=P, hid=P, nrm=P,
             T=16000, scale=1.0, peps=1e-6, neps=1e-6, sx=1.0, sr=1.0, hp=1, hn=1, stream=None)
    a.update(over)
    return mf.lib.beam_moe_finalize_norm_residual_norm(
        a["e"], a["cap"], a["K"], a["H"], a["w"], a["wrows"], a["res"], a["pw"], a["nw"], a["hid"],
        a["nrm"], a["T"], a["scale"], a["peps"], a["neps"], a["sx"], a["sr"], a["hp"], a["hn"],
        a["stream"])


@pytest.mark.parametrize("over,want", [
    (dict(T=0), OK), (dict(T=0, e=None, w=None, res=None, hid=None, nrm=None), OK),
    (dict(K=0), SHAPE), (dict(K=33), SHAPE), (dict(H=2100), SHAPE), (dict(T=16385), SHAPE),
    (dict(wrows=15999), SHAPE), (dict(cap=-1), SHAPE), (dict(T=-1), SHAPE),
    (dict(hp=0), ARG), (dict(hn=0), ARG),
    (dict(e=None), NULLP), (dict(w=None), NULLP), (dict(res=None), NULLP), (dict(hid=None), NULLP),
    (dict(nrm=None), NULLP), (dict(res=P + 2), ALIGN), (dict(nw=P + 2), ALIGN),
    (dict(hid=P + 8), ALIGN), (dict(nrm=P + 4), ALIGN), (dict(e=P + 2), ALIGN),
])
def test_fused_residual_norm_validation(over, want):
    assert fused_rn(**over) == want


def consumer(**over):
    a = dict(x=P, stride=2048, res=P, pw=None, nw=P, hid=P, nrm=P, T=100, H=2048, peps=0.0,
             neps=1e-6, sx=1.0, sr=1.0, hp=0, hn=1, stream=None)
    a.update(over)
    return mf.lib.beam_norm_residual_norm(
        a["x"], a["stride"], a["res"], a["pw"], a["nw"], a["hid"], a["nrm"], a["T"], a["H"],
        a["peps"], a["neps"], a["sx"], a["sr"], a["hp"], a["hn"], a["stream"])


@pytest.mark.parametrize("over,want", [
    (dict(T=0), OK), (dict(T=0, hn=0, nw=None, nrm=None, x=None, res=None, hid=None), OK),
    (dict(H=100), SHAPE), (dict(stride=1024), SHAPE), (dict(stride=2052), ALIGN),
    (dict(pw=P), ARG), (dict(hn=0), ARG), (dict(x=None), NULLP), (dict(res=None), NULLP),
    (dict(hid=None), NULLP), (dict(nrm=None), NULLP), (dict(x=P + 2), ALIGN),
])
def test_consumer_validation(over, want):
    assert consumer(**over) == want


def test_binding_rejects_host_tensors():
    import torch
    g = torch.zeros(8, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mf.moe_finalize(g, torch.zeros(1, 8), torch.zeros(1, 8, dtype=torch.int32),
                        torch.zeros(1, 256, dtype=torch.bfloat16))


def test_c_driver_links_against_the_library():
    """The plain-C driver of the GPU tests resolves libmoe_finalize.so and the
    HIP runtime; without arguments it prints its usage before any HIP call."""
    import subprocess
    driver = os.path.join(ROOT, "tests", "capi_c_driver")
    assert os.path.exists(driver), "run __graft_entry__.build() first"
    r = subprocess.run([driver], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage:" in r.stderr
