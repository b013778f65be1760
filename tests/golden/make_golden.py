"""Write tests/golden/oracle_digests.json: SHA-256 digests (and the first
eight values) of the CPU oracle's outputs on small seeded cases.

The finalize pages print no worked numeric example, so nothing here comes
from them; these fixtures only freeze the oracle's current outputs, so that
any later change to its arithmetic shows up as a failing test and has to be
justified (by the passage, or the reading of it, that requires it).  This
script calls only the oracle and the input generators.

    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads as wl  # noqa: E402


def cases():
    t = wl.tiny(poison=True)
    yield "tiny/moe_finalize_rmsnorm", oracle.moe_finalize_rmsnorm(
        t.gemm2, t.expert_weights, t.idx, t.norm_weight, eps=t.eps, gain_center=t.gain_center,
        weight_before_norm=t.weight_before_norm)
    yield "tiny/moe_finalize", oracle.moe_finalize(t.gemm2, t.expert_weights, t.idx, t.hidden)
    d = wl.decode(num_tokens=32, num_rows=256, poison=True)
    yield "decode32/moe_finalize_rmsnorm", oracle.moe_finalize_rmsnorm(
        d.gemm2, d.expert_weights, d.idx, d.norm_weight, eps=d.eps, gain_center=d.gain_center,
        weight_before_norm=d.weight_before_norm)
    yield "decode32/rmsnorm_of_finalize", oracle.rmsnorm(
        oracle.moe_finalize(d.gemm2, d.expert_weights, d.idx, d.hidden), d.norm_weight,
        eps=d.eps, gain_center=d.gain_center, weight_before_norm=d.weight_before_norm)
    b4 = wl.beam4(capacity=24, live_tokens=20)
    yield "beam4_small/beam_moe_finalize", oracle.beam_moe_finalize(
        b4.expert_outputs, b4.expert_weights, b4.live_tokens, b4.routed_scale)
    b5 = wl.beam5(capacity=40, live_tokens=33)
    yield "beam5_small/beam_moe_finalize", oracle.beam_moe_finalize(
        b5.expert_outputs, b5.expert_weights, b5.live_tokens, b5.routed_scale, b5.post_weight,
        b5.post_eps)
    rng = np.random.Generator(np.random.PCG64(77))
    res = wl.normal_bf16(rng, (33, 2048))
    nw = wl.normal_bf16(rng, (2048,), mean=1.0, std=0.1)
    h, n = oracle.beam_moe_finalize_norm_residual_norm(
        b5.expert_outputs, b5.expert_weights, res, b5.post_weight, b5.post_eps, nw, 1e-6,
        (0.5, 2.0), b5.routed_scale)
    yield "beam5_small/residual_hidden", h
    yield "beam5_small/residual_normalized", n


def digest(a: np.ndarray) -> dict:
    a = np.ascontiguousarray(a)
    return {"shape": list(a.shape), "sha256": hashlib.sha256(a.tobytes()).hexdigest(),
            "head": [f"{int(v):#06x}" for v in a.reshape(-1)[:8]]}


def compute() -> dict:
    return {name: digest(out) for name, out in cases()}


if __name__ == "__main__":
    path = os.path.join(HERE, "oracle_digests.json")
    with open(path, "w") as f:
        json.dump(compute(), f, indent=1)
    print("wrote", path)
