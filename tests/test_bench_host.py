"""Host-side logic of bench.py (no GPU): the multi-GPU refusal, the
algorithmic byte counts the roofline divides by, the ulp distance used for
its GPU-vs-oracle agreement figure, and the check that a stored traffic
record belongs to the current kernel sources."""
from __future__ import annotations

import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

import bench
from oracle_pins import bf16_ulp_distance

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def index_map_shape(T, K, H, weights_dtype, invalid=0, num_rows=None):
    idx = np.zeros((T, K), np.int32)
    idx.reshape(-1)[:invalid] = -1
    return SimpleNamespace(idx=idx, num_rows=num_rows or T * K, weights_dtype=weights_dtype,
                           num_tokens=T, top_k=K, hidden=H)


@pytest.mark.parametrize("T,K,H,wdt,expected", [
    # per token: K rows of H BF16 in, H BF16 out, K int32 indices, K weights;
    # plus the norm weight once: 8192*8*8192 + 8192*8192 + 8192*8*8 + 8192
    (8192, 8, 4096, "fp32", 604_512_256),
    (3000, 8, 7168, "fp32", 387_278_336),
    (16000, 16, 2048, "fp32", 1_116_164_096),
])
def test_index_map_bytes(T, K, H, wdt, expected):
    assert bench.index_map_bytes(index_map_shape(T, K, H, wdt), norm=True) == expected


def test_index_map_bytes_skip_invalid_slots_and_count_bf16_weights():
    c = index_map_shape(256, 8, 4096, "bf16", invalid=41)
    valid = 256 * 8 - 41
    assert bench.index_map_bytes(c, norm=True) == (valid * 4096 * 2 + 256 * 4096 * 2
                                                    + 256 * 8 * (4 + 2) + 4096 * 2)
    assert bench.index_map_bytes(c, norm=False) == bench.index_map_bytes(c, norm=True) - 8192


@pytest.mark.parametrize("L,K,H,post,expected", [
    (3000, 8, 7168, False, 387_168_000),
    (16000, 16, 2048, True, 1_115_140_096),
])
def test_token_major_bytes(L, K, H, post, expected):
    c = SimpleNamespace(live_tokens=L, top_k=K, hidden=H,
                        post_weight=np.zeros(H, np.uint16) if post else None)
    assert bench.token_major_bytes(c) == expected


def test_ulp_distance_matches_the_tests_definition():
    rng = np.random.Generator(np.random.PCG64(3))
    a = rng.integers(0, 1 << 16, size=200_000).astype(np.uint16)
    b = (a.astype(np.int64) + rng.integers(-3, 4, size=a.size)).astype(np.uint16)
    special = np.array([0x0000, 0x8000, 0x7FC0, 0xFFC1, 0x7F80, 0xFF80, 0x0001, 0x8001],
                       np.uint16)
    a = np.concatenate([a, special, special])
    b = np.concatenate([b, special[::-1], special])
    assert np.array_equal(bench.bf16_ulp_distance(a, b), bf16_ulp_distance(a, b))
    assert bench.bf16_ulp_distance(np.array([0x8000], np.uint16),
                                   np.array([0x0000], np.uint16))[0] == 0
    assert bench.bf16_ulp_distance(np.array([0x8001], np.uint16),
                                   np.array([0x0001], np.uint16))[0] == 2


def test_stored_traffic_requires_matching_sources(monkeypatch):
    path = os.path.join(ROOT, "profiles", "traffic_prefill.json")
    with open(path) as f:
        rec = json.load(f)
    monkeypatch.setattr(bench, "source_digest", lambda: rec["source_digest"])
    assert bench.stored_traffic("prefill") == rec["bytes_per_launch"]
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 16)
    assert bench.stored_traffic("prefill") is None
    assert bench.stored_traffic("no_such_workload") is None



def test_threaded_oracle_baseline_covers_every_token():
    """The all-cores CPU baseline splits the tokens into contiguous slices;
    the slices' outputs put together equal one pass over all tokens."""
    import oracle
    import workloads as wl
    c = wl.tiny(num_tokens=37, num_rows=37 * 8, invalid_frac=0.1)
    fake = SimpleNamespace(c=c, tokens=c.num_tokens)
    fake.cpu_oracle = lambda orc, sl: bench.IndexMapBench.cpu_oracle(fake, orc, sl)
    rec = bench.cpu_baseline_threads(fake, oracle, 0.0)
    assert rec["cores"] >= 1 and rec["value"] > 0 and rec["unit"] == "tokens/s"
    whole = fake.cpu_oracle(oracle, slice(0, 37))[0]
    parts = [fake.cpu_oracle(oracle, slice(a, b))[0] for a, b in ((0, 5), (5, 20), (20, 37))]
    assert np.array_equal(np.concatenate(parts), whole)


def test_agreement_stats():
    got = np.array([0x3F80, 0x3F81, 0x7FC0, 0x0000, 0x4000], np.uint16)
    want = np.array([0x3F80, 0x3F80, 0x3F80, 0x8000, 0x4002], np.uint16)
    a = bench.agreement_stats([(got, want)])
    assert a["elements"] == 5 and a["nan_outputs"] == 1
    assert a["max_ulp"] == 1 << 20                       # NaN against a number
    assert a["bit_exact_fraction"] == 2 / 5              # 0x3F80 and +0 == -0
    assert a["within_1_ulp_fraction"] == 3 / 5


@pytest.mark.parametrize("config,ratio", [
    (dict(T=8192, K=8, H=4096, kind="index"), 8),
    (dict(T=16000, K=16, H=2048, kind="token"), 16),
    (dict(T=3000, K=8, H=7168, kind="token"), 8),
    (dict(T=16000, K=16, H=2048, kind="residual"), 8),
])
def test_practical_ceiling_uses_the_workloads_mix(config, ratio):
    """The mixed probe reads as many vectors per write as the workload does
    (nearest of 4, 8, 16): 8 at top-k 8, 16 at top-k 16, and 8.5 -> 8 for the
    residual variant, which also reads the residual and writes two rows."""
    T, K, H = config["T"], config["K"], config["H"]
    if config["kind"] == "index":
        fake = SimpleNamespace(c=index_map_shape(T, K, H, "fp32"))
        fake.bytes = bench.index_map_bytes(fake.c, norm=True)
        r = bench.IndexMapBench.read_write_ratio(fake)
    elif config["kind"] == "token":
        fake = SimpleNamespace(c=SimpleNamespace(live_tokens=T, top_k=K, hidden=H,
                                                 post_weight=None))
        fake.bytes = bench.token_major_bytes(fake.c)
        r = bench.TokenMajorBench.read_write_ratio(fake)
    else:
        fake = SimpleNamespace(c=SimpleNamespace(live_tokens=T, top_k=K, hidden=H))
        fake.bytes = T * K * H * 2 + T * H * 2 * 3 + T * K * 4 + 2 * H * 2
        r = bench.ResidualBench.read_write_ratio(fake)
    assert bench.probe_ratio(r) == ratio

