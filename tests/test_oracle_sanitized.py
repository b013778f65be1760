"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer:
tests/oracle_asan_driver.c calls every entry point on small inputs with the
edge cases, built together with oracle/oracle.c by gcc."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "driver")
        cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-ffp-contract=off", os.path.join(HERE, "oracle_asan_driver.c"),
               os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe]
        b = subprocess.run(cmd, capture_output=True, text=True)
        if b.returncode != 0 and "asan" in (b.stderr + b.stdout).lower():
            pytest.skip("gcc has no sanitizer runtime here: " + b.stderr[-200:])
        assert b.returncode == 0, b.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert r.returncode == 0, r.stdout + r.stderr
        assert r.stdout.startswith("ok")
