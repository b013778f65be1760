"""Seeded random cases across the whole envelope, each run through the C ABI
and compared with the oracle element by element.

Every case draws its own hidden size (256..8192 in steps of 256), top-k
(1..32), token count, row-stride padding, weight dtype, logit spread, share
and kind of out-of-range indices (-1, -2, INT32_MIN, INT32_MAX, num_rows,
num_rows + 1, with and without NaN rows allocated behind num_rows), value
magnitude (rows scaled by 2^e, from FP32 subnormal sums to 2^40), norm
placement, gain_center, eps, routed_scale, live-token count and the post /
next norm options of the residual path.  Sizes are bounded so that the
oracle finishes a case in a fraction of a second; every case has at least
4096 output elements so that the bit-exact share floors mean something.

A second family draws small rows (hidden 256 and 512, top-k up to 8) with
up to 3000 tokens.

The bar is the fixed cases' bar: outputs without a norm are bit-exact,
normalised outputs within 1 BF16 ulp of the oracle.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import moe_expert_output_finalize_amd as mf
import oracle
import workloads as wl
from gpu_util import (NORM_MIN_EXACT, IndexMapOnDevice, TokenMajorOnDevice, check_residual,
                      dev_bf16, gpu_beam, gpu_finalize, gpu_rmsnorm, host_bits, oracle_beam,
                      oracle_finalize, oracle_rmsnorm, residual_case, sync)
from oracle_pins import assert_bits_equal, assert_within_ulp

pytestmark = pytest.mark.gpu

KINDS = ("index_map", "token_major", "residual", "standalone")
N_CASES = 64
N_SMALL_CASES = 64
MAX_GATHERED = 3_000_000          # gathered row elements per case
MIN_OUTPUT = 4096                 # output elements per case
INT32_MIN, INT32_MAX = int(np.iinfo(np.int32).min), int(np.iinfo(np.int32).max)


def draw_shape(rng, top_k_max=32, small=False):
    """(hidden, top-k, tokens).  small: hidden 256 or 512 at top-k up to 8,
    where one wave holds several tokens, with up to 3000 tokens so that the
    grid spans full runs of workgroups per XCD."""
    if small:
        hidden = 256 * int(rng.integers(1, 3))
        top_k = int(rng.integers(1, min(top_k_max, 8) + 1))
    else:
        hidden = 256 * int(rng.integers(1, 33))
        top_k = int(rng.integers(1, top_k_max + 1))
    t_min = math.ceil(MIN_OUTPUT / hidden)
    t_max = max(t_min, min(3000 if small else 300, MAX_GATHERED // (top_k * hidden)))
    return hidden, top_k, int(rng.integers(t_min, t_max + 1))


def draw_exponent(rng) -> int:
    return int(rng.choice([0, 0, 0, -130, -24, 8, 40]))


def scale_bits(bits: np.ndarray, e: int) -> np.ndarray:
    """BF16 bits times 2^e (NaN stays NaN); an input transform, not the method."""
    if e == 0:
        return bits
    return wl.to_bf16_bits(np.ldexp(wl.bf16_bits_to_f32(bits), e))


def describe(**kw) -> str:
    return " ".join(f"{k}={v}" for k, v in kw.items())


def run_index_map(seed, rng, small=False):
    H, K, T = draw_shape(rng, small=small)
    R = T * K + int(rng.integers(0, 64))
    S = H + 8 * int(rng.integers(0, 17))
    wdt = str(rng.choice(["fp32", "bf16"]))
    bad = float(rng.choice([0.0, 0.02, 0.2, 1.0]))
    nan_rows = int(rng.choice([0, 2]))
    wbn = bool(rng.integers(0, 2))
    gc = float(rng.choice([1.0, 0.0, -0.5, 2.0 ** -12]))
    eps = float(rng.choice([1e-6, 1e-5]))
    e = draw_exponent(rng)
    what = describe(seed=seed, H=H, K=K, T=T, R=R, S=S, w=wdt, invalid=bad, nan_rows=nan_rows,
                    wbn=wbn, gc=gc, eps=eps, exp=e)
    print(what, flush=True)
    c = wl.make_index_map_case(50_000 + seed, num_tokens=T, hidden=H, top_k=K, num_rows=R,
                               row_stride=S, weights_dtype=wdt,
                               logit_std=float(rng.choice([0.5, 1.0, 3.0])),
                               invalid_frac=bad, poison=True, nan_rows_beyond=nan_rows,
                               eps=eps, gain_center=gc, weight_before_norm=wbn)
    c.gemm2_storage = scale_bits(c.gemm2_storage, e)
    # other out-of-range values for about half of the invalid slots
    invalid = (c.idx < 0) | (c.idx >= R)
    pick = invalid & (rng.random(c.idx.shape) < 0.5)
    others = np.array([-1, -2, INT32_MIN, INT32_MAX, R, R + 1], dtype=np.int64)
    c.idx[pick] = rng.choice(others, size=int(pick.sum())).astype(np.int32)
    d = IndexMapOnDevice(c)
    want_f = oracle_finalize(c)
    assert_bits_equal(gpu_finalize(d), want_f, f"finalize {what}")
    assert_within_ulp(gpu_rmsnorm(d), oracle_rmsnorm(c), 1, NORM_MIN_EXACT, f"rmsnorm {what}")
    # unfused: the BF16 intermediate is the finalize output, then the norm
    mid = d.new_output()
    mf.moe_finalize(d.gemm2, d.weights, d.idx, mid)
    out = d.new_output()
    mf.mf_rmsnorm(mid, d.norm_weight, out, eps=eps, gain_center=gc, weight_before_norm=wbn)
    sync()
    assert_bits_equal(host_bits(mid), want_f, f"unfused intermediate {what}")
    want_n = oracle.rmsnorm(want_f, c.norm_weight, eps=eps, gain_center=gc,
                            weight_before_norm=wbn)
    assert_within_ulp(host_bits(out), want_n, 1, NORM_MIN_EXACT, f"unfused norm {what}")


def run_token_major(seed, rng, small=False):
    H, K, T = draw_shape(rng, small=small)
    cap = T + int(rng.integers(0, 5))
    norm = bool(rng.random() < 0.6)
    pw = (0.05 if rng.random() < 0.5 else None) if norm else None
    eps = float(rng.choice([1e-6, 1e-5])) if norm else None
    scale = float(rng.choice([1.0, 2.5, 0.3, 1.0 / 3.0, 16.0]))
    weights = str(rng.choice(["softmax", "uniform"]))
    e = draw_exponent(rng)
    live = T if rng.random() < 0.7 else int(rng.integers(math.ceil(T / 2), T + 1))
    what = describe(seed=seed, H=H, K=K, cap=cap, live=live, norm=norm, pw=pw, eps=eps,
                    scale=scale, weights=weights, exp=e)
    print(what, flush=True)
    c = wl.make_token_major_case(60_000 + seed, capacity=cap, top_k=K, hidden=H,
                                 live_tokens=T, weights=weights, routed_scale=scale,
                                 post_eps=eps, post_weight_std=pw, poison_dead=True)
    c.expert_outputs = scale_bits(c.expert_outputs, e)
    d = TokenMajorOnDevice(c)
    got, want = gpu_beam(d, live), oracle_beam(c, live)
    if norm:
        assert_within_ulp(got, want, 1, NORM_MIN_EXACT, what)
    else:
        assert_bits_equal(got, want, what)


def run_residual(seed, rng, small=False):
    H, K, T = draw_shape(rng, small=small)
    post = bool(rng.integers(0, 2))
    post_w = post and bool(rng.integers(0, 2))
    nxt = bool(rng.random() < 0.75)
    next_w = nxt and bool(rng.integers(0, 2))
    scales = [None, (0.5, 2.0), (1.5, -0.75), (1.0, 1.0)][int(rng.integers(0, 4))]
    routed = float(rng.choice([1.0, 2.5, 0.75]))
    what = describe(seed=seed, H=H, K=K, T=T, post=post, post_w=post_w, next=nxt,
                    next_w=next_w, scales=scales, routed_scale=routed)
    print(what, flush=True)
    args = residual_case(70_000 + seed, T + int(rng.integers(0, 3)), K, H, T, post, post_w,
                         nxt, next_w, scales, routed)
    check_residual(*args, what)


def run_standalone(seed, rng, small=False):
    """mf_rmsnorm and the residual consumer (no post-norm) on strided rows."""
    H, _, T = draw_shape(rng, top_k_max=1, small=small)
    S = H + 8 * int(rng.integers(0, 17))
    wbn = bool(rng.integers(0, 2))
    gc = float(rng.choice([1.0, 0.0, -0.5]))
    eps = float(rng.choice([1e-6, 1e-5]))
    e = draw_exponent(rng)
    next_w = bool(rng.integers(0, 2))
    scales = [None, (0.5, 2.0), (1.5, -0.75)][int(rng.integers(0, 3))]
    what = describe(seed=seed, H=H, T=T, S=S, wbn=wbn, gc=gc, eps=eps, exp=e, next_w=next_w,
                    scales=scales)
    print(what, flush=True)
    x = wl.normal_bf16(rng, (T, S))
    x[:, H:] = 0x7FC0                                  # padding is never read
    x = scale_bits(x, e)
    nw = wl.normal_bf16(rng, (H,), mean=1.0, std=0.1)
    res = wl.normal_bf16(rng, (T, H))
    xd, nwd, resd = dev_bf16(x)[:, :H], dev_bf16(nw), dev_bf16(res)
    out = xd.new_empty((T, H))
    mf.mf_rmsnorm(xd, nwd, out, eps=eps, gain_center=gc, weight_before_norm=wbn)
    h, n = mf.beam_norm_residual_norm(xd, resd, None, None, nwd if next_w else None, eps,
                                      scales)
    sync()
    want = oracle.rmsnorm(x, nw, eps=eps, gain_center=gc, weight_before_norm=wbn)
    assert_within_ulp(host_bits(out), want, 1, NORM_MIN_EXACT, f"mf_rmsnorm {what}")
    wh, wn = oracle.beam_norm_residual_norm(x, res, None, None, nw if next_w else None, eps,
                                            scales)
    assert_bits_equal(host_bits(h), wh, f"consumer hidden {what}")
    assert_within_ulp(host_bits(n), wn, 1, NORM_MIN_EXACT, f"consumer normalized {what}")


RUNNERS = {"index_map": run_index_map, "token_major": run_token_major,
           "residual": run_residual, "standalone": run_standalone}


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_case(seed):
    kind = KINDS[seed % len(KINDS)]
    rng = np.random.Generator(np.random.PCG64(40_000 + seed))
    RUNNERS[kind](seed, rng)


# Small rows (hidden 256 and 512, top-k up to 8): the kernels that hold
# several tokens per wave, and beside them the one-token kernels of the same
# hidden sizes.
@pytest.mark.parametrize("seed", range(N_SMALL_CASES))
def test_random_small_row_case(seed):
    kind = KINDS[seed % len(KINDS)]
    rng = np.random.Generator(np.random.PCG64(90_000 + seed))
    RUNNERS[kind](1000 + seed, rng, small=True)
