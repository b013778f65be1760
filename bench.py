#!/usr/bin/env python3
"""Throughput of the MoE finalize hot path on one MI355X.

A step is one launch of the fused finalize over one batch of synthetic input
resident in HBM.  The default workload is the prefill finalize+RMSNorm
(8192 tokens, hidden 4096, top-k 8, FP32 weights, 65536 gathered rows grouped
by expert with Zipf(1.1) load over 256 experts).  To keep the gathered rows
from being served by the 256 MB Infinity Cache, steps rotate over several
device copies of the row matrix and output (at least 1.5 GiB in total), so
every step reads its rows from HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config prefill]
    python bench.py --envelope        (the fused kernel over hidden x top-k)

Prints one JSON line on stdout (diagnostics go to stderr): tokens/s over the
timed region, the dominant kernel's achieved HBM bandwidth against the
8 TB/s peak (a pair of HIP events on the launch stream around the timed
back-to-back launches), the fused kernel against the unfused two-kernel
baseline, and the CPU oracle's throughput on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
MAX_CPU_THREADS = 16                # the host share of one GPU
ROTATE_MIN_BYTES = 3 << 29          # 1.5 GiB of rotated rows + outputs

WORKLOADS = {
    "prefill": "prefill finalize+RMSNorm: 8192 tokens, hidden 4096, top-k 8, FP32 weights, "
               "65536 rows grouped by expert (Zipf 1.1 over 256 experts)",
    "decode": "decode finalize+RMSNorm: 256 tokens, hidden 4096 (row stride 4160), top-k 8, "
              "BF16 weights, 2% invalid slots, weight before norm",
    "tiny": "tiny finalize+RMSNorm: 16 tokens, hidden 4096, top-k 8, 5% invalid slots",
    "beam4": "token-major finalize, no norm: 3000 live of 4096, top-k 8, hidden 7168, scale 2.5",
    "beam5": "token-major finalize + post RMSNorm: 16000 live of 16384, top-k 16, hidden 2048",
    "beam5_residual": "token-major finalize + post RMSNorm + residual add + next RMSNorm: "
                      "16000 of 16384 tokens, top-k 16, hidden 2048",
    "imap7168": "index-map finalize+RMSNorm: 3000 tokens, hidden 7168, top-k 8, FP32 weights, "
                "24000 rows grouped by expert (Zipf 1.1 over 256 experts)",
    "imap2048k16": "index-map finalize+RMSNorm (weight before norm): 16000 tokens, hidden 2048, "
                   "top-k 16, FP32 weights, 256000 rows grouped by expert (Zipf 1.1 over 256)",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="prefill", choices=sorted(WORKLOADS))
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip timing the CPU oracle (profiling runs)")
    p.add_argument("--no-probes", action="store_true",
                   help="skip the memory-system probes and the per-dispatch pass "
                        "(profiling runs)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU time spent on the oracle sample")
    p.add_argument("--graph", action="store_true",
                   help="capture the timed steps in one HIP graph and replay it (for "
                        "launch-bound small workloads)")
    p.add_argument("--envelope", action="store_true",
                   help="instead of one workload, time the fused kernel over a grid of "
                        "hidden sizes and top-k on both layouts")
    p.add_argument("--shapes", default="",
                   help="with --envelope: only these comma-separated layout:hidden:top_k "
                        "cells, e.g. index_map:7168:32,token_major:7168:32")
    p.add_argument("--tokens", default="",
                   help="with --envelope: comma-separated token counts to run each cell "
                        "at, instead of the count that gives ~256 MiB of gathered rows")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="only run a plain device copy of this size (counter calibration)")
    return p.parse_args()


def source_digest() -> str:
    """Digest of the library's sources and flags (the one its build records)."""
    import importlib.util
    path = os.path.join(ROOT, "moe_expert_output_finalize_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_mf_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.source_digest(ROOT)[:16]


def stored_traffic(config: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{config}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        log(f"bench: {path} was measured on other kernel sources; traffic = null")
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------ workloads -----

def index_map_bytes(c, norm: bool) -> int:
    valid = int(((c.idx >= 0) & (c.idx < c.num_rows)).sum())
    wbytes = 4 if c.weights_dtype == "fp32" else 2
    T, K, H = c.num_tokens, c.top_k, c.hidden
    return valid * H * 2 + T * H * 2 + T * K * 4 + T * K * wbytes + (H * 2 if norm else 0)


def token_major_bytes(c) -> int:
    L, K, H = c.live_tokens, c.top_k, c.hidden
    return L * K * H * 2 + L * H * 2 + L * K * 4 + (H * 2 if c.post_weight is not None else 0)


class IndexMapBench:
    def __init__(self, c, torch, mf):
        import numpy as np
        self.c, self.torch, self.mf = c, torch, mf
        dev = torch.device("cuda:0")
        self.tokens = c.num_tokens
        self.bytes = index_map_bytes(c, norm=True)
        per_set = c.num_rows * c.row_stride * 2 + c.num_tokens * c.hidden * 2
        self.sets = max(2, math.ceil(ROTATE_MIN_BYTES / per_set))
        g = torch.from_numpy(c.gemm2.view(np.int16)).view(torch.bfloat16).to(dev)
        self.rows = [g] + [g.clone() for _ in range(self.sets - 1)]
        self.outs = [torch.empty((c.num_tokens, c.hidden), dtype=torch.bfloat16, device=dev)
                     for _ in range(self.sets)]
        w = c.expert_weights
        self.w = (torch.from_numpy(w.view(np.int16)).view(torch.bfloat16)
                  if w.dtype == np.uint16 else torch.from_numpy(w)).to(dev)
        self.idx = torch.from_numpy(c.idx).to(dev)
        self.nw = torch.from_numpy(c.norm_weight.view(np.int16)).view(torch.bfloat16).to(dev)

    def step(self, i: int):
        s = i % self.sets
        c = self.c
        self.mf.moe_finalize_rmsnorm(self.rows[s], self.w, self.idx, self.nw, self.outs[s],
                                     eps=c.eps, gain_center=c.gain_center,
                                     weight_before_norm=c.weight_before_norm)

    # The unfused baseline: moe_finalize into a BF16 intermediate, then the
    # standalone norm (two launches, one extra write and read of [T, H]).
    def unfused_parts(self):
        c, torch = self.c, self.torch
        mids = [torch.empty_like(o) for o in self.outs]
        outs = [torch.empty_like(o) for o in self.outs]

        def finalize(i):
            s = i % self.sets
            self.mf.moe_finalize(self.rows[s], self.w, self.idx, mids[s])

        def norm(i):
            s = i % self.sets
            self.mf.mf_rmsnorm(mids[s], self.nw, outs[s], eps=c.eps,
                               gain_center=c.gain_center,
                               weight_before_norm=c.weight_before_norm)
        extra = 2 * c.num_tokens * c.hidden * 2
        return [("moe_finalize", finalize), ("mf_rmsnorm", norm)], self.bytes + extra

    def cpu_oracle(self, oracle, tokens: slice):
        c = self.c
        return [oracle.moe_finalize_rmsnorm(c.gemm2, c.expert_weights[tokens], c.idx[tokens],
                                            c.norm_weight, eps=c.eps, gain_center=c.gain_center,
                                            weight_before_norm=c.weight_before_norm)]

    def gpu_outputs(self):
        return [self.outs[0]]

    def read_write_ratio(self) -> float:
        w = self.c.num_tokens * self.c.hidden * 2
        return (self.bytes - w) / w


class TokenMajorBench:
    def __init__(self, c, torch, mf):
        import numpy as np
        self.c, self.torch, self.mf = c, torch, mf
        dev = torch.device("cuda:0")
        self.tokens = c.live_tokens
        self.bytes = token_major_bytes(c)
        per_set = c.expert_outputs.nbytes + c.live_tokens * c.hidden * 2
        self.sets = max(2, math.ceil(ROTATE_MIN_BYTES / per_set))
        e = torch.from_numpy(c.expert_outputs.view(np.int16)).view(torch.bfloat16).to(dev)
        self.rows = [e] + [e.clone() for _ in range(self.sets - 1)]
        self.outs = [torch.empty((c.live_tokens, c.hidden), dtype=torch.bfloat16, device=dev)
                     for _ in range(self.sets)]
        self.w = torch.from_numpy(c.expert_weights).to(dev)
        self.pw = (None if c.post_weight is None else
                   torch.from_numpy(c.post_weight.view(np.int16)).view(torch.bfloat16).to(dev))

    def step(self, i: int):
        s = i % self.sets
        c = self.c
        self.mf.beam_moe_finalize(self.rows[s], self.w, self.outs[s], c.routed_scale, self.pw,
                                  c.post_eps)

    def cpu_oracle(self, oracle, tokens: slice):
        c = self.c
        n = len(range(*tokens.indices(c.live_tokens)))
        return [oracle.beam_moe_finalize(c.expert_outputs[tokens], c.expert_weights[tokens], n,
                                         c.routed_scale, c.post_weight, c.post_eps)]

    def gpu_outputs(self):
        return [self.outs[0]]

    def read_write_ratio(self) -> float:
        w = self.c.live_tokens * self.c.hidden * 2
        return (self.bytes - w) / w


def time_launches(torch, fns, steps: int, warmup: int):
    """Time `steps` steps, each running the functions in `fns` back to back.
    Returns the step time (us) from one HIP-event pair around all steps,
    the wall time per step (ms), and each function's share (us) from event
    pairs around every launch, which read 1-3 us high per launch."""
    for i in range(warmup):
        for _, fn in fns:
            fn(i)
    torch.cuda.synchronize()
    s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s0.record()
    for i in range(steps):
        for _, fn in fns:
            fn(warmup + i)
    e0.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    step_us = s0.elapsed_time(e0) * 1e3 / steps
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in fns] for _ in range(steps)]
    for i in range(steps):
        for (s, e), (_, fn) in zip(ev[i], fns):
            s.record()
            fn(warmup + steps + i)
            e.record()
    torch.cuda.synchronize()
    us = {name: sum(ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(steps)) / steps * 1e3
          for j, (name, _) in enumerate(fns)}
    return step_us, wall_ms, us


class ResidualBench(TokenMajorBench):
    """beam_moe_finalize_norm_residual_norm on the beam5 shape: post-norm,
    residual add and next norm fused into the finalize."""

    def __init__(self, c, torch, mf):
        import numpy as np
        import workloads as wl
        super().__init__(c, torch, mf)
        rng = np.random.Generator(np.random.PCG64(5))
        L, H = c.live_tokens, c.hidden
        dev = torch.device("cuda:0")
        res = wl.normal_bf16(rng, (L, H))
        nw = wl.normal_bf16(rng, (H,), mean=1.0, std=0.1)
        self.res_host, self.nw_host = res, nw
        self.res = torch.from_numpy(res.view(np.int16)).view(torch.bfloat16).to(dev)
        self.nw = torch.from_numpy(nw.view(np.int16)).view(torch.bfloat16).to(dev)
        self.outs2 = [torch.empty_like(o) for o in self.outs]
        self.next_eps = 1e-6
        # gather + residual + hidden + normalized + weights + both norm weights
        self.bytes = (L * c.top_k * H * 2 + L * H * 2 * 3 + L * c.top_k * 4 + 2 * H * 2)

    def step(self, i: int):
        s = i % self.sets
        c = self.c
        self.mf.beam_moe_finalize_norm_residual_norm(
            self.rows[s], self.w, self.res, self.pw, c.post_eps, self.nw, self.next_eps, None,
            c.routed_scale, hidden_out=self.outs[s], normalized_out=self.outs2[s])

    def read_write_ratio(self) -> float:
        w = 2 * self.c.live_tokens * self.c.hidden * 2     # hidden and normalized
        return (self.bytes - w) / w

    # The page's unfused strategy: beam_moe_finalize, then the consumer.
    def unfused_parts(self):
        c, torch = self.c, self.torch
        mids = [torch.empty_like(o) for o in self.outs]
        hid = [torch.empty_like(o) for o in self.outs]
        nrm = [torch.empty_like(o) for o in self.outs]
        self.unfused_outputs = (mids, hid, nrm)

        def finalize(i):
            s = i % self.sets
            self.mf.beam_moe_finalize(self.rows[s], self.w, mids[s], c.routed_scale, self.pw,
                                      c.post_eps)

        def consumer(i):
            s = i % self.sets
            self.mf.beam_norm_residual_norm(mids[s], self.res, None, None, self.nw,
                                            self.next_eps, None, hidden_out=hid[s],
                                            normalized_out=nrm[s])
        extra = 2 * c.live_tokens * c.hidden * 2
        return [("beam_moe_finalize", finalize), ("beam_norm_residual_norm", consumer)], \
            self.bytes + extra

    def cpu_oracle(self, oracle, tokens: slice):
        c = self.c
        return list(oracle.beam_moe_finalize_norm_residual_norm(
            c.expert_outputs[tokens], c.expert_weights[tokens], self.res_host[tokens],
            c.post_weight, c.post_eps, self.nw_host, self.next_eps, None, c.routed_scale))

    def gpu_outputs(self):
        return [self.outs[0], self.outs2[0]]

    def agreement(self, oracle) -> dict:
        """The parity tests' criterion, stage by stage, on the whole workload:
        y (the finalize step of the unfused path, set 0) against the oracle's
        finalize; the fused kernel's hidden and normalized (set 0) against the
        oracle's consumer applied to that y; and the fused outputs against the
        unfused path's, bit for bit.  (Comparing the fused outputs with the
        oracle's fused op directly is not a valid test after a post-norm:
        where hidden = y + residual nearly cancels, the one-ulp freedom of y
        is many ulps of hidden.)"""
        import numpy as np
        c = self.c
        mids, hid, nrm = self.unfused_outputs

        def bits(t):
            return t.cpu().view(self.torch.int16).numpy().view(np.uint16)

        y = bits(mids[0])
        want_y = oracle.beam_moe_finalize(c.expert_outputs, c.expert_weights, c.live_tokens,
                                          c.routed_scale, c.post_weight, c.post_eps)
        want_h, want_n = oracle.beam_norm_residual_norm(y, self.res_host, None, None,
                                                        self.nw_host, self.next_eps, None)
        got_h, got_n = bits(self.outs[0]), bits(self.outs2[0])
        stages = {"finalize_y_vs_oracle": agreement_stats([(y, want_y)]),
                  "fused_hidden_vs_oracle_consumer_of_y": agreement_stats([(got_h, want_h)]),
                  "fused_normalized_vs_oracle_consumer_of_y": agreement_stats([(got_n,
                                                                              want_n)])}
        stages["fused_equals_unfused"] = bool(np.array_equal(got_h, bits(hid[0])) and
                                              np.array_equal(got_n, bits(nrm[0])))
        stages["max_ulp"] = max(v["max_ulp"] for v in stages.values() if isinstance(v, dict))
        stages["criterion"] = ("each stage within 1 ulp; fused == unfused bit for bit "
                               "(the parity tests' check)")
        return stages


def bf16_ulp_distance(a, b):
    """Distance in BF16 grid steps between two uint16 bit-pattern arrays
    (+0 == -0; NaN vs NaN is 0, NaN vs a number is 2^20)."""
    import numpy as np
    a = a.astype(np.int64)
    b = b.astype(np.int64)

    def ordered(v):
        return np.where(v & 0x8000, -(v & 0x7FFF), v & 0x7FFF)

    d = np.abs(ordered(a) - ordered(b))
    na = ((a & 0x7F80) == 0x7F80) & ((a & 0x7F) != 0)
    nb = ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    return np.where(na | nb, np.where(na & nb, 0, 1 << 20), d)


def agreement_stats(pairs) -> dict:
    """Element-wise agreement of (GPU bits, oracle bits) pairs: the largest
    BF16 ulp distance, the bit-exact and within-1-ulp shares, and how many
    GPU outputs are NaN."""
    import numpy as np
    worst, exact, within1, n, nans = 0, 0, 0, 0, 0
    for got, want in pairs:
        d = bf16_ulp_distance(got, want)
        worst = max(worst, int(d.max()))
        exact += int((d == 0).sum())
        within1 += int((d <= 1).sum())
        nans += int((((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)).sum())
        n += d.size
    return {"max_ulp": worst, "bit_exact_fraction": exact / max(n, 1),
            "within_1_ulp_fraction": within1 / max(n, 1), "elements": n, "nan_outputs": nans}


def cpu_baseline(bench, seconds: float) -> dict:
    """The oracle (single-threaded C) on whole passes over the workload's
    tokens, repeated until `seconds` of CPU time have been spent.  Its output
    is also compared with what the timed GPU steps wrote."""
    import numpy as np
    import oracle
    oracle.build()
    T = bench.tokens
    reps, t0 = 0, time.perf_counter()
    first = None
    while True:
        out = bench.cpu_oracle(oracle, slice(0, T))
        first = out if first is None else first
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    if hasattr(bench, "agreement"):
        agree = bench.agreement(oracle)
    else:
        agree = agreement_stats([(got.cpu().view(bench.torch.int16).numpy().view(np.uint16), want)
                                 for want, got in zip(first, bench.gpu_outputs())])
    agree["unread_inputs"] = "NaN (padding columns, dead tokens)"
    return {"value": reps * T / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full pass(es) over all {T} tokens of the same workload, "
                      f"single thread, {el:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0)), "host_cpu": cpu_model(),
            "all_cores": cpu_baseline_threads(bench, oracle, seconds),
            "gpu_vs_oracle": agree}


def cpu_baseline_threads(bench, oracle, seconds: float) -> dict:
    """The same oracle over all host cores: each pass splits the tokens into
    one contiguous slice per thread (the oracle's C code runs without the
    interpreter lock), repeated until `seconds` have passed."""
    from concurrent.futures import ThreadPoolExecutor
    T = bench.tokens
    n = max(1, min(MAX_CPU_THREADS, len(os.sched_getaffinity(0)), T))
    bounds = [T * i // n for i in range(n + 1)]
    slices = [slice(bounds[i], bounds[i + 1]) for i in range(n)]
    reps, t0 = 0, time.perf_counter()
    with ThreadPoolExecutor(max_workers=n) as pool:
        while True:
            list(pool.map(lambda sl: bench.cpu_oracle(oracle, sl), slices))
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": reps * T / el, "unit": "tokens/s", "cores": n,
            "sample": f"{reps} full pass(es) over all {T} tokens, {n} threads on "
                      f"contiguous token slices, {el:.1f} s"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def copy_probe(torch, mib: int = 1024, reps: int = 10) -> float:
    """GB/s (read + write) of torch's device-to-device copy: the known-size
    kernel the HBM traffic counters are calibrated on."""
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del a, b
    return 2 * n / (ms * 1e-3) / 1e9


# ------------------------------------------------- memory-system ceilings --

PROBE_BLOCKS = (1024, 2048, 4096, 8192)   # grid-stride probes: workgroups of 256
PROBE_POLICIES = (0, 2, 16)        # store cache policy: default, nt, sc1
PROBE_BYTES = 1 << 30              # per probe: far beyond the 256 MB Infinity Cache


def load_probes():
    """libmf_probes.so (csrc/bench_probes.hip): streaming read, write and
    mixed read:write kernels, not part of the finalize ABI."""
    import ctypes
    path = os.path.join(ROOT, "moe_expert_output_finalize_amd", "libmf_probes.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build()")
    so = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    so.mf_probe_read.argtypes = [vp, i64, vp, i32, i32, vp]
    so.mf_probe_write.argtypes = [vp, i64, i32, i32, i32, vp]
    so.mf_probe_mixed.argtypes = [vp, vp, i64, i32, i32, i32, i32, vp]
    so.mf_probe_rows.argtypes = [i32, i32, i32, vp, vp, vp, i64, i32, i64, vp]
    for f in (so.mf_probe_read, so.mf_probe_write, so.mf_probe_mixed, so.mf_probe_rows):
        f.restype = i32
    return so


PROBE_TEAMS = (256, 512)
PROBE_RESIDENT = (0, 2, 4, 8)      # workgroups per CU the row probes allow (0: no cap)


def probe_ratio(read_write_ratio: float) -> int:
    """The mixed probe's reads per write nearest (in ratio) to the workload's."""
    return min((4, 8, 16), key=lambda r: abs(math.log(r / max(read_write_ratio, 1e-9))))


def memory_ceilings(torch, read_write_ratio: float, reps: int = 10) -> dict:
    """Best GB/s of streaming probes in this run, for three traffic mixes:
    read only, write only, and reads and writes in the workload's own
    proportion (rounded to 4, 8 or 16 reads per write).  Two probe shapes
    are tried over launch shapes, residency caps and store cache policies:
    grid-stride loops (PROBE_BLOCKS workgroups of 256 threads), and the
    finalize's own shape of work without its arithmetic (one workgroup per
    token reading `ratio` contiguous rows of team x 16 bytes, all in flight,
    and writing one row; teams PROBE_TEAMS, PROBE_RESIDENT workgroups per
    CU).  The mixed figure is the practical ceiling for the kernel's traffic:
    the same mix with every access contiguous."""
    so = load_probes()
    stream = torch.cuda.current_stream().cuda_stream
    ratio = probe_ratio(read_write_ratio)
    n16 = PROBE_BYTES // 16
    src = torch.empty(PROBE_BYTES, dtype=torch.uint8, device="cuda")
    src.random_(0, 255)
    dst = torch.empty(PROBE_BYTES, dtype=torch.uint8, device="cuda")
    flag = torch.zeros(64, dtype=torch.int32, device="cuda")
    lds_cu = getattr(torch.cuda.get_device_properties(0), "shared_memory_per_multiprocessor",
                     160 * 1024)

    def rate(go, nbytes):
        rc = go()
        assert rc == 0, f"probe launch failed ({rc})"
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            go()
        e1.record()
        torch.cuda.synchronize()
        return nbytes / (e0.elapsed_time(e1) * 1e-3 / reps) / 1e9

    best = {"read": (0.0, ""), "write": (0.0, ""), "mixed": (0.0, "")}

    def keep(mode, gbps, how):
        if gbps > best[mode][0]:
            best[mode] = (gbps, how)

    out16 = n16 // ratio
    for blocks in PROBE_BLOCKS:
        keep("read", rate(lambda: so.mf_probe_read(src.data_ptr(), n16, flag.data_ptr(), blocks,
                                                   256, stream), PROBE_BYTES),
             f"grid-stride, {blocks} x 256")
        for pol in PROBE_POLICIES:
            keep("write", rate(lambda: so.mf_probe_write(dst.data_ptr(), n16, pol, blocks, 256,
                                                         stream), PROBE_BYTES),
                 f"grid-stride, {blocks} x 256, store policy {pol}")
            keep("mixed", rate(lambda: so.mf_probe_mixed(src.data_ptr(), dst.data_ptr(), out16,
                                                         ratio, pol, blocks, 256, stream),
                               out16 * 16 * (ratio + 1)),
                 f"grid-stride, {blocks} x 256, store policy {pol}")
    for team in PROBE_TEAMS:
        tokens = PROBE_BYTES // (ratio * team * 16)
        for resident in PROBE_RESIDENT:
            lds = lds_cu // resident - 1024 if resident else 0
            where = f"one token per workgroup of {team}, {resident or 'uncapped'} per CU"
            keep("read", rate(lambda: so.mf_probe_rows(0, ratio, 0, src.data_ptr(), None,
                                                       flag.data_ptr(), tokens, team, lds,
                                                       stream), tokens * ratio * team * 16),
                 where)
            for pol in PROBE_POLICIES:
                keep("write", rate(lambda: so.mf_probe_rows(1, ratio, pol, None, dst.data_ptr(),
                                                            None, tokens, team, lds, stream),
                                   tokens * ratio * team * 16), f"{where}, store policy {pol}")
                keep("mixed", rate(lambda: so.mf_probe_rows(2, ratio, pol, src.data_ptr(),
                                                            dst.data_ptr(), None, tokens, team,
                                                            lds, stream),
                                   tokens * (ratio + 1) * team * 16),
                     f"{where}, store policy {pol}")
    del src, dst, flag
    torch.cuda.empty_cache()
    return {"read_only_GBps": best["read"][0], "write_only_GBps": best["write"][0],
            "mixed_GBps": best["mixed"][0], "mixed_reads_per_write": ratio,
            "best_shapes": {k: v[1] for k, v in best.items()},
            "bytes_per_probe": PROBE_BYTES,
            "note": "best of probe shapes, residency caps and store cache policies, same run"}


def dispatch_stats(torch, step, first: int, steps: int) -> dict:
    """Per-dispatch kernel time from a pair of HIP events around each of
    `steps` launches (a separate pass from the headline's back-to-back span:
    the events between launches add a gap of their own, so these read a
    little high)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record()
        step(first + i)
        b.record()
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    return {"median_us": us[len(us) // 2], "min_us": us[0], "max_us": us[-1],
            "mean_us": sum(us) / len(us), "dispatches": len(us)}


ENVELOPE_HIDDEN = (256, 512, 1024, 2048, 4096, 7168, 8192)
ENVELOPE_TOPK = (1, 2, 4, 6, 8, 12, 16, 32)
ENVELOPE_ROW_BYTES = 256 << 20      # gathered row bytes per launch (before rotation)
ENVELOPE_MAX_TOKENS = 1 << 17       # hidden 256 at top-k 1-2, 512 at 1: 64-128 MiB of rows
ENVELOPE_SPANS = 5


def envelope(torch, mf, wl, steps: int, warmup: int, shapes: str = "",
             tokens: str = "") -> dict:
    """Fused kernel time over hidden x top-k on both layouts: index map
    (expert-grouped Zipf 1.1 map, FP32 weights, RMSNorm) and token major
    (post-norm).  Inputs are seeded N(0,1) rows made on the device; the
    token count gives about 256 MiB of gathered rows per launch (at most
    ENVELOPE_MAX_TOKENS tokens, so hidden 256 at top-k 1 and 2 and hidden
    512 at top-k 1 carry 64-128 MiB), and steps
    rotate over copies totalling at least 1.5 GiB, as in the main bench.  A
    cell's time is the median of ENVELOPE_SPANS spans of steps / ENVELOPE_SPANS
    back-to-back launches.  The rows are drawn in BF16 in place and every
    cell's buffers are released before the next, so no cell runs in memory
    left fragmented by a larger one's temporaries."""
    import numpy as np
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    results = []
    cells = [(layout, H, K) for layout in ("index_map", "token_major")
             for H in ENVELOPE_HIDDEN for K in ENVELOPE_TOPK]
    if shapes:
        cells = []
        for item in shapes.split(","):
            layout, H, K = item.split(":")
            assert layout in ("index_map", "token_major"), layout
            cells.append((layout, int(H), int(K)))
    for layout, H, K in cells:
        counts = ([int(t) for t in tokens.split(",")] if tokens else
                  [max(256, min(ENVELOPE_MAX_TOKENS, ENVELOPE_ROW_BYTES // (K * H * 2)))])
        for T in counts:
            gen.manual_seed(1000 * H + K)
            rng = np.random.Generator(np.random.PCG64(1000 * H + K))
            w = torch.from_numpy(wl.softmax_rows(rng.standard_normal((T, K)) * 2.0)).to(dev)
            nw = (torch.randn(H, generator=gen, device=dev) * 0.1).to(torch.bfloat16)
            rows = torch.empty((T * K, H), dtype=torch.bfloat16, device=dev)
            rows.normal_(generator=gen)
            per_set = rows.numel() * 2 + T * H * 2
            sets = max(2, math.ceil(ROTATE_MIN_BYTES / per_set))
            rs = [rows] + [rows.clone() for _ in range(sets - 1)]
            outs = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(sets)]
            if layout == "index_map":
                idx = torch.from_numpy(wl.zipf_grouped_index_map(rng, T, K, 256, 1.1)).to(dev)
                nbytes = T * K * H * 2 + T * H * 2 + T * K * 8 + H * 2

                def step(i):
                    mf.moe_finalize_rmsnorm(rs[i % sets], w, idx, nw, outs[i % sets],
                                            eps=1e-6, gain_center=1.0,
                                            weight_before_norm=False)
            else:
                rs = [r.view(T, K, H) for r in rs]
                nbytes = T * K * H * 2 + T * H * 2 + T * K * 4 + H * 2

                def step(i):
                    mf.beam_moe_finalize(rs[i % sets], w, outs[i % sets], 1.0, nw, 1e-6)
            for i in range(warmup):
                step(i)
            torch.cuda.synchronize()
            # ENVELOPE_SPANS spans of back-to-back launches, the events of
            # consecutive spans recorded between launches with no wait in
            # between (the GPU never idles, as in the headline's single
            # span); the median span, so one disturbed span does not decide.
            per = max(1, steps // ENVELOPE_SPANS)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(ENVELOPE_SPANS + 1)]
            ev[0].record()
            for r in range(ENVELOPE_SPANS):
                for i in range(per):
                    step(warmup + r * per + i)
                ev[r + 1].record()
            torch.cuda.synchronize()
            spans = [ev[r].elapsed_time(ev[r + 1]) * 1e3 / per for r in range(ENVELOPE_SPANS)]
            us = sorted(spans)[len(spans) // 2]
            gbps = nbytes / us / 1e3
            results.append({"layout": layout, "hidden": H, "top_k": K, "tokens": T,
                            "kernel_us": us, "GBps": gbps, "frac": gbps / PEAK_HBM_GBPS})
            log(f"bench: envelope {layout} H={H} K={K} T={T}: {us:.2f} us, "
                f"{gbps:.0f} GB/s ({100 * gbps / PEAK_HBM_GBPS:.1f} %)")
            del rs, outs, rows
            torch.cuda.empty_cache()
    fr = sorted(r["frac"] for r in results)
    return {"metric": "achieved HBM GB/s of the fused finalize over the hidden x top-k envelope",
            "value": fr[len(fr) // 2] * PEAK_HBM_GBPS, "unit": "GB/s", "statistic": "median",
            "min_frac": fr[0], "median_frac": fr[len(fr) // 2], "max_frac": fr[-1],
            "n_gpus": 1, "steps": steps, "warmup": warmup, "higher_is_better": True,
            "data": "synthetic", "shapes": results}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: "
              "the finalize is per token and needs no communication, so each GPU runs "
              "it on its own share of the tokens and the one-GPU figure is that share's",
              file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.copy_probe_mib:
        log(f"bench: copy probe of {args.copy_probe_mib} MiB")
        gbps = copy_probe(torch, args.copy_probe_mib, reps=5)
        print(json.dumps({"copy_probe_mib": args.copy_probe_mib, "GBps": gbps}))
        return

    import moe_expert_output_finalize_amd as mf
    import workloads as wl

    if args.envelope:
        print(json.dumps(envelope(torch, mf, wl, args.steps, args.warmup, args.shapes,
                                  args.tokens)), flush=True)
        return

    log(f"bench: generating the {args.config} workload")
    # What is never read is filled with NaN (padding columns, rows and weights
    # of tokens past the live count), so the oracle comparison at the end also
    # shows that nothing leaks; it costs nothing, being never read.
    if args.config == "beam5_residual":
        c = wl.beam5(poison_dead=True)
        bench = ResidualBench(c, torch, mf)
    elif args.config in ("beam4", "beam5"):
        c = wl.CONFIGS[args.config](poison_dead=True)
        bench = TokenMajorBench(c, torch, mf)
    else:
        c = wl.CONFIGS[args.config](poison=True)
        bench = IndexMapBench(c, torch, mf)
    log(f"bench: {bench.sets} rotating buffer sets, {bench.bytes} algorithmic bytes/step")

    for i in range(args.warmup):
        bench.step(i)
    torch.cuda.synchronize()

    # Timed region: K back-to-back launches on the current stream, bracketed
    # by synchronisation (wall clock) and by one pair of HIP events recorded
    # on that same stream (kernel time per launch = event span / K).  With
    # --graph the K launches are captured once in a HIP graph and the timed
    # region is one replay of it.
    K = args.steps
    graph = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            bench.step(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(K):
                bench.step(args.warmup + i)
        graph.replay()
        torch.cuda.synchronize()
    ev_start = torch.cuda.Event(enable_timing=True)
    ev_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_start.record()
    if graph is not None:
        graph.replay()
    else:
        for i in range(K):
            bench.step(args.warmup + i)
    ev_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_avg_s = ev_start.elapsed_time(ev_end) * 1e-3 / K

    achieved = bench.bytes / kern_avg_s / 1e9
    # Secondary figure: the same launches all on one buffer set, so part of
    # the rows may come from the Infinity Cache.  Never the headline.
    torch.cuda.synchronize()
    hot_start = torch.cuda.Event(enable_timing=True)
    hot_end = torch.cuda.Event(enable_timing=True)
    hot_start.record()
    for _ in range(K):
        bench.step(0)
    hot_end.record()
    torch.cuda.synchronize()
    hot_us = hot_start.elapsed_time(hot_end) * 1e3 / K
    traffic = stored_traffic(args.config)
    dispatch, ceil = None, None
    if not args.no_probes:
        dispatch = dispatch_stats(torch, bench.step, args.warmup + K, K)
        dispatch["span_mean_us"] = kern_avg_s * 1e6
        dispatch["note"] = ("event pair around each launch in a separate pass; the gaps the "
                            "events add make these read high by about mean_us - span_mean_us")
        ceil = memory_ceilings(torch, bench.read_write_ratio())
        log(f"bench: per dispatch median {dispatch['median_us']:.2f} us, min "
            f"{dispatch['min_us']:.2f} us; ceilings read {ceil['read_only_GBps']:.0f}, write "
            f"{ceil['write_only_GBps']:.0f}, {ceil['mixed_reads_per_write']}:1 mix "
            f"{ceil['mixed_GBps']:.0f} GB/s")
    log(f"bench: kernel avg {kern_avg_s * 1e6:.2f} us, {achieved:.0f} GB/s; "
        f"wall {wall * 1e3 / K:.3f} ms/step")

    unfused = None
    if hasattr(bench, "unfused_parts"):
        parts, unfused_bytes = bench.unfused_parts()
        step_us, wall_ms, us = time_launches(torch, parts, K, args.warmup)
        unfused = {"step_us": step_us, "kernels_us": us,
                   "kernels_us_note": "event pair around each launch: 1-3 us high each",
                   "ms_per_step": wall_ms,
                   "algorithmic_bytes_per_step": unfused_bytes,
                   "achieved_GBps": unfused_bytes / (step_us * 1e-6) / 1e9,
                   "fused_speedup": step_us / (kern_avg_s * 1e6)}
        log(f"bench: unfused baseline {step_us:.2f} us per step ({us}) -> fused is "
            f"{unfused['fused_speedup']:.2f}x faster")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"bench: timing the CPU oracle for >= {args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(bench, args.cpu_seconds)

    config = {"workload": WORKLOADS[args.config], "name": args.config,
              "launch": "hip_graph" if args.graph else "stream",
              "tokens_per_step": bench.tokens, "algorithmic_bytes_per_step": bench.bytes,
              "rotating_buffer_sets": bench.sets, "io_dtype": "bf16"}
    if isinstance(c, wl.IndexMapCase):
        config.update(hidden=c.hidden, top_k=c.top_k, num_rows=c.num_rows,
                      row_stride=c.row_stride, weights=c.weights_dtype)
    else:
        config.update(hidden=c.hidden, top_k=c.top_k, capacity=c.capacity)
    rec = {
        "metric": "tokens/sec and achieved HBM GB/s (% of peak), finalize+RMSNorm h=4096 k=8",
        "value": bench.tokens * K / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": config,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": traffic, "kernel_avg_us": kern_avg_s * 1e6,
                     "frac_of_practical_ceiling": achieved / ceil["mixed_GBps"] if ceil else None,
                     "practical_ceiling": ceil, "dispatch": dispatch},
        "cpu_baseline": cpu,
        "unfused_baseline": unfused,
        "hot_cache": {"kernel_avg_us": hot_us, "GBps": bench.bytes / hot_us / 1e3,
                      "note": "every launch on the same buffers (rows may hit the "
                              "Infinity Cache); secondary, not the headline"},
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
