"""Argument tables for the host-side tests of the C ABI.

Each entry point's parameters are listed in prototype order with a kind
(p pointer, L int64_t, i int32_t, f float) and a valid default.  A case is
(entry point, overrides, expected status): the defaults with the named
arguments replaced.  The pointers are fake 16-byte-aligned addresses that
the host-only builds these cases run against never dereference.

The same cases run two ways: through ctypes against the host-check library
(the C ABI's host code linked with a recording stand-in for the GPU
launcher, tests/capi_host_stub.cpp) and through tests/capi_sanitize_driver.c
built with AddressSanitizer and UndefinedBehaviorSanitizer.
"""
from __future__ import annotations

import ctypes

OK, NULLP, SHAPE, DTYPE, ALIGN, ARG, LAUNCH = 0, 1, 2, 3, 4, 5, 6
BF16, FP32 = 1, 2
P = 0x10000              # a 16-byte aligned fake device address
INT32_MAX = 2 ** 31 - 1
INT64_MAX = 2 ** 63 - 1

SIGNATURES = {
    "moe_finalize_rmsnorm": [
        ("g", "p", P), ("rows", "L", 128), ("stride", "L", 4096), ("w", "p", P),
        ("wdt", "i", FP32), ("idx", "p", P), ("nw", "p", P), ("out", "p", P), ("T", "L", 16),
        ("H", "i", 4096), ("K", "i", 8), ("eps", "f", 1e-6), ("gc", "f", 1.0), ("wbn", "i", 0),
        ("stream", "p", 0)],
    "moe_finalize": [
        ("g", "p", P), ("rows", "L", 128), ("stride", "L", 4096), ("w", "p", P),
        ("wdt", "i", FP32), ("idx", "p", P), ("out", "p", P), ("T", "L", 16), ("H", "i", 4096),
        ("K", "i", 8), ("stream", "p", 0)],
    "beam_moe_finalize": [
        ("e", "p", P), ("cap", "L", 4096), ("K", "i", 8), ("H", "i", 7168), ("w", "p", P),
        ("wrows", "L", 4096), ("out", "p", P), ("live", "L", 3000), ("pw", "p", 0),
        ("scale", "f", 2.5), ("eps", "f", 0.0), ("norm", "i", 0), ("stream", "p", 0)],
    "mf_rmsnorm": [
        ("x", "p", P), ("stride", "L", 4096), ("nw", "p", P), ("out", "p", P), ("T", "L", 16),
        ("H", "i", 4096), ("eps", "f", 1e-6), ("gc", "f", 1.0), ("wbn", "i", 0),
        ("stream", "p", 0)],
    "beam_moe_finalize_norm_residual_norm": [
        ("e", "p", P), ("cap", "L", 16384), ("K", "i", 16), ("H", "i", 2048), ("w", "p", P),
        ("wrows", "L", 16384), ("res", "p", P), ("pw", "p", P), ("nw", "p", P),
        ("hid", "p", P), ("nrm", "p", P), ("T", "L", 16000), ("scale", "f", 1.0),
        ("peps", "f", 1e-6), ("neps", "f", 1e-6), ("sx", "f", 1.0), ("sr", "f", 1.0),
        ("hp", "i", 1), ("hn", "i", 1), ("stream", "p", 0)],
    "beam_norm_residual_norm": [
        ("x", "p", P), ("stride", "L", 2048), ("res", "p", P), ("pw", "p", 0), ("nw", "p", P),
        ("hid", "p", P), ("nrm", "p", P), ("T", "L", 100), ("H", "i", 2048), ("peps", "f", 0.0),
        ("neps", "f", 1e-6), ("sx", "f", 1.0), ("sr", "f", 1.0), ("hp", "i", 0), ("hn", "i", 1),
        ("stream", "p", 0)],
}

_CTYPES = {"p": ctypes.c_void_p, "L": ctypes.c_int64, "i": ctypes.c_int32,
           "f": ctypes.c_float}


def _cases(fn, rows):
    return [(fn, over, want) for over, want in rows]


# Each case is valid but for the named change.
CASES = (
    _cases("moe_finalize_rmsnorm", [
        (dict(), OK), (dict(T=0), OK),
        (dict(T=0, g=None, w=None, idx=None, nw=None, out=None), OK),
        (dict(H=2048, K=4), OK), (dict(H=256, K=1), OK), (dict(H=8192, K=32, stride=8192), OK),
        (dict(rows=0, g=None), OK), (dict(wdt=BF16, wbn=1), OK),
        (dict(H=2000), SHAPE), (dict(H=8448, stride=8448), SHAPE), (dict(K=0), SHAPE),
        (dict(K=33), SHAPE), (dict(T=-1), SHAPE), (dict(rows=-1), SHAPE),
        (dict(T=1 << 31), SHAPE), (dict(stride=4088), SHAPE),
        (dict(rows=2, stride=INT64_MAX - 7), SHAPE),
        (dict(stride=4100), ALIGN), (dict(wdt=0), DTYPE), (dict(wdt=3), DTYPE),
        (dict(g=None), NULLP), (dict(w=None), NULLP), (dict(idx=None), NULLP),
        (dict(nw=None), NULLP), (dict(out=None), NULLP),
        (dict(g=P + 2), ALIGN), (dict(w=P + 4), ALIGN), (dict(idx=P + 8), ALIGN),
        (dict(nw=P + 2), ALIGN), (dict(out=P + 8), ALIGN),
    ]) +
    _cases("moe_finalize", [
        (dict(), OK), (dict(T=0), OK), (dict(T=0, H=256, K=1), OK),
        (dict(T=0, H=8192, K=32, stride=8192), OK), (dict(T=0, rows=0, g=None), OK),
        (dict(H=768, K=13, stride=776), OK),
        (dict(H=128), SHAPE), (dict(H=8448, stride=8448), SHAPE), (dict(H=4000), SHAPE),
        (dict(K=0), SHAPE), (dict(K=33), SHAPE), (dict(stride=2048, H=4096), SHAPE),
        (dict(stride=4100), ALIGN), (dict(wdt=7), DTYPE),
        (dict(out=None), NULLP), (dict(g=None), NULLP), (dict(g=P + 4), ALIGN),
    ]) +
    _cases("beam_moe_finalize", [
        (dict(), OK), (dict(live=0), OK), (dict(live=0, e=None, w=None, out=None), OK),
        (dict(live=0, norm=1, pw=P, eps=1e-6), OK), (dict(norm=1, pw=P, eps=1e-6), OK),
        (dict(norm=1, eps=1e-6), OK), (dict(cap=INT64_MAX, wrows=INT64_MAX), OK),
        (dict(K=0), SHAPE), (dict(K=33), SHAPE), (dict(H=7000), SHAPE), (dict(H=0), SHAPE),
        (dict(H=8448), SHAPE), (dict(live=4097), SHAPE), (dict(wrows=2999), SHAPE),
        (dict(cap=-1), SHAPE), (dict(live=-1), SHAPE),
        (dict(pw=P, norm=0), ARG), (dict(e=None), NULLP), (dict(w=None), NULLP),
        (dict(out=None), NULLP), (dict(e=P + 8), ALIGN), (dict(w=P + 2), ALIGN),
        (dict(out=P + 2), ALIGN), (dict(pw=P + 2, norm=1), ALIGN),
    ]) +
    _cases("mf_rmsnorm", [
        (dict(), OK), (dict(T=0), OK), (dict(T=0, x=None, nw=None, out=None), OK),
        (dict(T=0, H=256), OK), (dict(stride=4160, wbn=1), OK),
        (dict(H=200), SHAPE), (dict(H=8448, stride=8448), SHAPE), (dict(T=-1), SHAPE),
        (dict(stride=4000), SHAPE), (dict(T=3, stride=INT64_MAX - 7), SHAPE),
        (dict(stride=4100), ALIGN),
        (dict(x=None), NULLP), (dict(nw=None), NULLP), (dict(out=None), NULLP),
        (dict(x=P + 2), ALIGN), (dict(nw=P + 8), ALIGN), (dict(out=P + 4), ALIGN),
    ]) +
    _cases("beam_moe_finalize_norm_residual_norm", [
        (dict(), OK), (dict(T=0), OK), (dict(T=0, e=None, w=None, res=None, hid=None, nrm=None), OK),
        (dict(hp=0, pw=None, hn=0, nw=None, nrm=None), OK),
        (dict(K=0), SHAPE), (dict(K=33), SHAPE), (dict(H=2100), SHAPE), (dict(T=16385), SHAPE),
        (dict(wrows=15999), SHAPE), (dict(cap=-1), SHAPE), (dict(T=-1), SHAPE),
        (dict(hp=0), ARG), (dict(hn=0), ARG),
        (dict(e=None), NULLP), (dict(w=None), NULLP), (dict(res=None), NULLP),
        (dict(hid=None), NULLP), (dict(nrm=None), NULLP), (dict(res=P + 2), ALIGN),
        (dict(nw=P + 2), ALIGN), (dict(hid=P + 8), ALIGN), (dict(nrm=P + 4), ALIGN),
        (dict(e=P + 2), ALIGN),
    ]) +
    _cases("beam_norm_residual_norm", [
        (dict(), OK), (dict(T=0), OK),
        (dict(T=0, hn=0, nw=None, nrm=None, x=None, res=None, hid=None), OK),
        (dict(H=100), SHAPE), (dict(stride=1024), SHAPE), (dict(stride=2052), ALIGN),
        (dict(T=5, stride=INT64_MAX - 7), SHAPE),
        (dict(pw=P), ARG), (dict(hn=0), ARG), (dict(x=None), NULLP), (dict(res=None), NULLP),
        (dict(hid=None), NULLP), (dict(nrm=None), NULLP), (dict(x=P + 2), ALIGN),
    ])
)

# Token counts whose launches must be split: (entry point, overrides,
# expected number of launches).  The work-items of one launch are capped at
# 2^31; the team is 512 threads at hidden 4096 on the index map (one vector
# per thread), 64 at hidden 256 (one wave holding four tokens at top-k 1, so
# 2^27 tokens per launch, and two at top-k 2, 2^26), 256 at token-major
# hidden 4096 (two vectors per thread), 448
# at 7168, and 512 for the standalone norm at hidden 8192 (two vectors per
# thread).
SPLIT_CASES = [
    ("moe_finalize_rmsnorm", dict(T=4_194_304), 1),
    ("moe_finalize_rmsnorm", dict(T=4_194_305), 2),
    ("moe_finalize_rmsnorm", dict(T=8_388_609), 3),
    ("moe_finalize", dict(T=INT32_MAX, H=256, stride=256, K=1), 16),
    ("moe_finalize", dict(T=134_217_728, H=256, stride=256, K=1), 1),
    ("moe_finalize", dict(T=134_217_729, H=256, stride=256, K=1), 2),
    ("moe_finalize", dict(T=67_108_864, H=256, stride=256, K=2), 1),
    ("moe_finalize", dict(T=67_108_865, H=256, stride=256, K=2), 2),
    ("moe_finalize", dict(T=INT32_MAX, H=512, stride=512, K=1), 32),
    ("moe_finalize", dict(T=67_108_865, H=512, stride=512, K=1), 2),
    ("beam_moe_finalize", dict(cap=INT32_MAX, wrows=INT32_MAX, live=INT32_MAX, H=4096), 256),
    ("beam_moe_finalize", dict(cap=10_000_000, wrows=10_000_000, live=4_793_491), 2),
    ("mf_rmsnorm", dict(T=INT32_MAX, H=8192, stride=8192), 512),
    ("mf_rmsnorm", dict(T=INT32_MAX, H=256, stride=256), 16),
    ("beam_norm_residual_norm", dict(T=INT32_MAX, H=256, stride=256), 16),
    ("beam_moe_finalize_norm_residual_norm",
     dict(cap=INT32_MAX, wrows=INT32_MAX, T=INT32_MAX, H=256, K=2), 32),
]


def values(fn: str, over: dict) -> list:
    sig = SIGNATURES[fn]
    unknown = set(over) - {n for n, _, _ in sig}
    assert not unknown, (fn, unknown)
    return [over.get(n, d) for n, _, d in sig]


def declare(lib) -> None:
    """Give every entry point of `lib` its ctypes prototype."""
    for fn, sig in SIGNATURES.items():
        f = getattr(lib, fn)
        f.argtypes = [_CTYPES[k] for _, k, _ in sig]
        f.restype = ctypes.c_int


def ctypes_call(lib, fn: str, over: dict) -> int:
    return getattr(lib, fn)(*values(fn, over))


def driver_line(fn: str, over: dict) -> str:
    out = [fn]
    for (name, kind, _), v in zip(SIGNATURES[fn], values(fn, over)):
        if kind == "p":
            out.append(str(0 if v is None else int(v)))
        elif kind == "f":
            out.append(repr(float(v)))
        else:
            out.append(str(int(v)))
    return " ".join(out)


def case_id(case) -> str:
    fn, over, want = case[0], case[1], case[2]
    return f"{fn}-" + ("-".join(f"{k}={v}" for k, v in over.items()) or "valid") + f"->{want}"
