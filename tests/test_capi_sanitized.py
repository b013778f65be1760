"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/capi_sanitize_driver.c, csrc/capi.cpp (the entry points' validation
and argument set-up, the same source the library is built from) and the
recording launcher stand-in of tests/capi_host_stub.cpp (which plans each
call's launches with csrc/plan.hpp) are built with gcc/g++ and both
sanitizers, with no recovery.  Every case of the host validation tests, the
launch splits of the largest token counts and a failed launch are fed to it
in one run; any sanitizer report fails the test, and every status must be
the documented one."""
import os
import shutil
import subprocess
import tempfile

import pytest

import capi_cases as cc

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "moe_expert_output_finalize_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def build_driver(d: str) -> str:
    exe = os.path.join(d, "capi_sanitize_driver")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src, cc_, std in ((os.path.join(CSRC, "capi.cpp"), "g++", "-std=c++17"),
                          (os.path.join(HERE, "capi_host_stub.cpp"), "g++", "-std=c++17"),
                          (os.path.join(HERE, "capi_sanitize_driver.c"), "gcc", "-std=c11")):
        obj = os.path.join(d, os.path.basename(src) + ".o")
        b = subprocess.run([cc_, std, *SAN, "-Wall", "-Wextra", *inc, "-c", src, "-o", obj],
                           capture_output=True, text=True)
        if b.returncode != 0 and "asan" in (b.stderr + b.stdout).lower():
            pytest.skip("no sanitizer runtime here: " + b.stderr[-200:])
        assert b.returncode == 0, b.stderr
        objs.append(obj)
    b = subprocess.run(["g++", *SAN, *objs, "-o", exe], capture_output=True, text=True)
    assert b.returncode == 0, b.stderr
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                    reason="needs gcc and g++")
def test_capi_host_code_clean_under_asan_ubsan():
    lines, want = [], []
    for fn, over, status in cc.CASES:
        lines += ["reset", cc.driver_line(fn, over)]
        want.append(("status", fn, over, status))
    for fn, over, launches in cc.SPLIT_CASES:
        lines += ["reset", cc.driver_line(fn, over)]
        want.append(("split", fn, over, launches))
    lines += ["reset", "fail 98", cc.driver_line("moe_finalize", {}),
              cc.driver_line("moe_finalize", {})]
    want += [("failed", "moe_finalize", {}, None), ("recovered", "moe_finalize", {}, None)]
    with tempfile.TemporaryDirectory() as d:
        exe = build_driver(d)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True,
                           text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]
    out = r.stdout.splitlines()
    assert len(out) == len(want)
    for line, (kind, fn, over, expect) in zip(out, want):
        v = [int(x) for x in line.split()]
        status, rec, has_msg = v[0], v[1:15], v[15]
        calls, launches, violations = rec[0], rec[10], rec[13]
        what = (kind, fn, over, line)
        assert violations == 0, what
        if kind == "status":
            assert status == expect, what
            zero = any(over.get(k) == 0 for k in ("T", "live"))
            assert calls == (1 if status == cc.OK and not zero else 0), what
        elif kind == "split":
            assert status == cc.OK and calls == 1 and launches == expect, what
        elif kind == "failed":
            assert status == cc.LAUNCH and has_msg == 1, what
        else:
            assert status == cc.OK and has_msg == 0, what
