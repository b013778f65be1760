"""The C ABI used from C: tests/capi_c_driver (built by __graft_entry__.build()
from capi_c_driver.c with gcc, the HIP runtime and include/moe_finalize.h
only) runs an index-map finalize with and without RMSNorm and a token-major
finalize on its own device buffers and stream, and checks the status codes
of invalid calls.  Its outputs are compared here with the oracle: no-norm
outputs bit-exact, the normalised output within 1 BF16 ulp."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import NORM_MIN_EXACT
from oracle_pins import assert_bits_equal, assert_within_ulp

pytestmark = pytest.mark.gpu

DRIVER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "capi_c_driver")


@pytest.mark.parametrize("wdt,wbn,gc", [("fp32", False, 1.0), ("bf16", True, 0.0)])
def test_c_program_uses_the_library(tmp_path, wdt, wbn, gc):
    if not os.path.exists(DRIVER):
        pytest.fail(f"{DRIVER} is missing: run __graft_entry__.build() first")
    c = wl.make_index_map_case(81, num_tokens=37, hidden=3072, top_k=6, num_rows=37 * 6 + 9,
                               row_stride=3072 + 64, weights_dtype=wdt, invalid_frac=0.1,
                               poison=True, eps=1e-5, gain_center=gc, weight_before_norm=wbn)
    b = wl.make_token_major_case(82, capacity=29, top_k=5, hidden=1280, live_tokens=29,
                                 weights="uniform", routed_scale=2.5)
    live = 23
    files = {"gemm2.bin": c.gemm2, "weights.bin": c.expert_weights, "idx.bin": c.idx,
             "norm_weight.bin": c.norm_weight, "beam_rows.bin": b.expert_outputs,
             "beam_weights.bin": b.expert_weights}
    for name, arr in files.items():
        np.ascontiguousarray(arr).tofile(tmp_path / name)
    args = [DRIVER, str(tmp_path), str(c.num_tokens), str(c.hidden), str(c.top_k),
            str(c.num_rows), str(c.row_stride), "1" if wdt == "bf16" else "2", repr(c.eps),
            repr(gc), str(int(wbn)), str(b.capacity), str(b.top_k), str(b.hidden), str(live),
            "2.5"]
    print(" ".join(args[2:]), flush=True)
    r = subprocess.run(args, capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "capi_c_driver: ok" in r.stdout

    def load(name, rows, cols):
        return np.fromfile(tmp_path / name, dtype=np.uint16).reshape(rows, cols)

    T, H = c.num_tokens, c.hidden
    assert_bits_equal(load("out_finalize.bin", T, H), oracle.moe_finalize(
        c.gemm2, c.expert_weights, c.idx, H), "C driver moe_finalize")
    want = oracle.moe_finalize_rmsnorm(c.gemm2, c.expert_weights, c.idx, c.norm_weight,
                                       eps=c.eps, gain_center=gc, weight_before_norm=wbn)
    assert_within_ulp(load("out_rmsnorm.bin", T, H), want, 1, NORM_MIN_EXACT,
                      "C driver moe_finalize_rmsnorm")
    assert_bits_equal(load("out_beam.bin", live, b.hidden), oracle.beam_moe_finalize(
        b.expert_outputs, b.expert_weights, live, 2.5), "C driver beam_moe_finalize")
