"""GPU parity: the HIP library (through the C ABI) against the CPU oracle,
element by element, on the same seeded inputs.

Bar: outputs without a norm (moe_finalize, beam_moe_finalize without
post-norm) are bit-exact, index masking included; normalised outputs are
within 1 BF16 ulp of the oracle's single rounding of the exact result.
Padding columns, rows past num_rows and rows of dead tokens hold NaN, so any
read the method does not make shows up as NaN in the output.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import moe_expert_output_finalize_amd as mf
import oracle
import workloads as wl
from gpu_util import (NORM_MIN_EXACT, IndexMapOnDevice, TokenMajorOnDevice, check_residual,
                      dev_bf16, gpu_beam, gpu_finalize, gpu_rmsnorm, host_bits, oracle_beam,
                      oracle_finalize, oracle_rmsnorm, residual_case, sync)
from oracle_pins import _f32_probe_values, assert_bits_equal, assert_within_ulp

pytestmark = pytest.mark.gpu

_cases = {}


def case(name, make):
    if name not in _cases:
        _cases[name] = make()
    return _cases[name]


# ------------------------------------------------------ the five configs ----

INDEX_CONFIGS = {
    "tiny": lambda: wl.tiny(poison=True),
    "tiny_nan_rows": lambda: wl.tiny(nan_rows_beyond=2),
    "decode": lambda: wl.decode(poison=True),
    "prefill": lambda: wl.prefill(),
    "imap7168": lambda: wl.imap7168(),
    "imap2048k16": lambda: wl.imap2048k16(),
}


@pytest.mark.parametrize("name", list(INDEX_CONFIGS))
def test_rmsnorm_config(name):
    c = case(name, INDEX_CONFIGS[name])
    d = IndexMapOnDevice(c)
    got = gpu_rmsnorm(d)
    want = oracle_rmsnorm(c)
    assert_within_ulp(got, want, 1, NORM_MIN_EXACT, f"{name} rmsnorm")
    # the other weight placement and weight dtype on the same inputs
    got = gpu_rmsnorm(d, weight_before_norm=not c.weight_before_norm)
    want = oracle_rmsnorm(c, weight_before_norm=not c.weight_before_norm)
    assert_within_ulp(got, want, 1, NORM_MIN_EXACT, f"{name} rmsnorm flipped placement")


@pytest.mark.parametrize("name", list(INDEX_CONFIGS))
def test_finalize_config(name):
    c = case(name, INDEX_CONFIGS[name])
    d = IndexMapOnDevice(c)
    assert_bits_equal(gpu_finalize(d), oracle_finalize(c), f"{name} finalize")


def test_rmsnorm_weight_dtypes():
    for wdt in ("fp32", "bf16"):
        c = wl.tiny(num_tokens=40, num_rows=400, weights_dtype=wdt, invalid_frac=0.1,
                    poison=True, nan_rows_beyond=3)
        d = IndexMapOnDevice(c)
        for wbn in (False, True):
            for gc in (1.0, 0.0, -0.5):
                got = gpu_rmsnorm(d, weight_before_norm=wbn, gain_center=gc)
                want = oracle_rmsnorm(c, weight_before_norm=wbn, gain_center=gc)
                assert_within_ulp(got, want, 1, NORM_MIN_EXACT, f"{wdt} wbn={wbn} gc={gc}")
        assert_bits_equal(gpu_finalize(d), oracle_finalize(c), f"{wdt} finalize")


BEAM_CONFIGS = {
    "beam4": lambda: wl.beam4(poison_dead=True),
    "beam5": lambda: wl.beam5(poison_dead=True),
}


@pytest.mark.parametrize("name", list(BEAM_CONFIGS))
def test_beam_config(name):
    c = case(name, BEAM_CONFIGS[name])
    d = TokenMajorOnDevice(c)
    got = gpu_beam(d)
    want = oracle_beam(c)
    if c.post_eps is None:
        assert_bits_equal(got, want, name)
    else:
        assert_within_ulp(got, want, 1, NORM_MIN_EXACT, name)


# ------------------------------------------------------- envelope sweeps ----

SWEEP_H = [256, 768, 1280, 2048, 3840, 4096, 7168, 8192]
# Each kernel variant at a full and a partly used slot count: run-time top-k
# sized for 2 slots (1, 2), 4 (3, 4), 8 (6, 7), 12 (9, 12), 16 (13), 24
# (17, 24) and 32 (25, 32), and compile-time 8 and 16.  Above 8 slots the
# rows arrive in one batch or through the rolling window, depending on the
# vectors per thread.  With the hidden sizes above this also covers one,
# two, four and eight vectors per thread and the half-idle last wave of odd
# hidden / 256.
SWEEP_K = [1, 2, 3, 4, 6, 7, 8, 9, 12, 13, 16, 17, 24, 25, 32]


@pytest.mark.parametrize("hidden", SWEEP_H)
def test_finalize_envelope(hidden):
    for K in SWEEP_K:
        for wdt in ("fp32", "bf16"):
            T = 11
            c = wl.make_index_map_case(1000 + hidden + K, num_tokens=T, hidden=hidden, top_k=K,
                                       num_rows=T * K + 5, row_stride=hidden + 8 * (K % 3),
                                       weights_dtype=wdt, invalid_frac=0.15, poison=True,
                                       nan_rows_beyond=2)
            d = IndexMapOnDevice(c)
            assert_bits_equal(gpu_finalize(d), oracle_finalize(c), f"H={hidden} K={K} {wdt}")


@pytest.mark.parametrize("hidden", SWEEP_H)
def test_rmsnorm_envelope(hidden):
    """Index-map finalize + RMSNorm over the whole hidden / top-k envelope."""
    for K in SWEEP_K:
        for wdt, wbn, gc in (("fp32", False, 1.0), ("bf16", True, 0.0), ("fp32", True, -0.5)):
            T = 11
            c = wl.make_index_map_case(3000 + hidden + K, num_tokens=T, hidden=hidden, top_k=K,
                                       num_rows=T * K + 5, row_stride=hidden + 8 * (K % 3),
                                       weights_dtype=wdt, invalid_frac=0.15, poison=True,
                                       nan_rows_beyond=2, weight_before_norm=wbn,
                                       gain_center=gc)
            d = IndexMapOnDevice(c)
            assert_within_ulp(gpu_rmsnorm(d), oracle_rmsnorm(c), 1, NORM_MIN_EXACT,
                              f"H={hidden} K={K} {wdt} wbn={wbn}")


@pytest.mark.parametrize("hidden", SWEEP_H)
def test_beam_envelope(hidden):
    for K in SWEEP_K:
        for norm, pw, scale in ((False, None, 1.75), (True, 0.05, 1.0), (True, None, 0.3)):
            c = wl.make_token_major_case(2000 + hidden + K, capacity=13, top_k=K, hidden=hidden,
                                         live_tokens=11, routed_scale=scale,
                                         post_eps=1e-6 if norm else None, post_weight_std=pw,
                                         poison_dead=True)
            d = TokenMajorOnDevice(c)
            got, want = gpu_beam(d), oracle_beam(c)
            what = f"H={hidden} K={K} norm={norm} pw={pw}"
            if norm:
                assert_within_ulp(got, want, 1, NORM_MIN_EXACT, what)
            else:
                assert_bits_equal(got, want, what)


# ----------------------------------------------- unfused baseline (f2) ------

def gpu_unfused(d: IndexMapOnDevice, **kw):
    """moe_finalize into a BF16 intermediate, then mf_rmsnorm."""
    c = d.case
    args = dict(eps=c.eps, gain_center=c.gain_center, weight_before_norm=c.weight_before_norm)
    args.update(kw)
    mid = d.new_output()
    mf.moe_finalize(d.gemm2, d.weights, d.idx, mid)
    out = d.new_output()
    mf.mf_rmsnorm(mid, d.norm_weight, out, **args)
    sync()
    return host_bits(mid), host_bits(out)


@pytest.mark.parametrize("name", list(INDEX_CONFIGS))
def test_unfused_pipeline_config(name):
    c = case(name, INDEX_CONFIGS[name])
    d = IndexMapOnDevice(c)
    mid, out = gpu_unfused(d)
    want_mid = oracle_finalize(c)
    assert_bits_equal(mid, want_mid, f"{name} unfused intermediate")
    want = oracle.rmsnorm(want_mid, c.norm_weight, eps=c.eps, gain_center=c.gain_center,
                          weight_before_norm=c.weight_before_norm)
    assert_within_ulp(out, want, 1, NORM_MIN_EXACT, f"{name} unfused norm")


@pytest.mark.parametrize("hidden", SWEEP_H)
def test_standalone_norm_envelope(hidden):
    rng = np.random.Generator(np.random.PCG64(4000 + hidden))
    T = 13
    x = wl.normal_bf16(rng, (T, hidden + 64))
    x[:, hidden:] = 0x7FC0                       # padding never read
    nw = wl.normal_bf16(rng, (hidden,), mean=1.0, std=0.1)
    xd, nwd = dev_bf16(x), dev_bf16(nw)
    for wbn, gc in ((False, 0.0), (True, 1.0), (False, -0.5)):
        out = torch.empty((T, hidden), dtype=torch.bfloat16, device="cuda")
        mf.mf_rmsnorm(xd[:, :hidden], nwd, out, eps=1e-5, gain_center=gc, weight_before_norm=wbn)
        sync()
        want = oracle.rmsnorm(x, nw, eps=1e-5, gain_center=gc, weight_before_norm=wbn)
        assert_within_ulp(host_bits(out), want, 1, NORM_MIN_EXACT, f"H={hidden} wbn={wbn}")


# ------------------------------- finalize -> residual -> next norm (f1) -----

def test_residual_norm_beam5_shape():
    """The beam5 shape (capacity 16384, top-k 16, hidden 2048) with a post-norm,
    the residual add and the next norm over 16000 tokens."""
    args = residual_case(61, 16384, 16, 2048, 16000, True, True, True, True, None)
    check_residual(*args, "beam5 post-norm")


@pytest.mark.parametrize("post,post_w,nxt,next_w,scales", [
    (False, False, False, False, None), (False, False, True, True, None),
    (True, False, True, False, None), (True, True, False, False, (0.5, 2.0)),
    (False, False, True, True, (1.5, -0.75)), (True, True, True, True, (1.0, 1.0)),
])
def test_residual_norm_options(post, post_w, nxt, next_w, scales):
    for hidden, K, scale in ((7168, 8, 2.5), (2048, 16, 1.0), (768, 3, 0.75), (8192, 1, 1.0),
                             (256, 1, 1.5), (256, 3, 1.0), (256, 16, 1.25)):
        args = residual_case(70 + hidden + K, 40, K, hidden, 33, post, post_w, nxt, next_w,
                             scales, scale)
        check_residual(*args, f"H={hidden} K={K} post={post} next={nxt} scales={scales}")


@pytest.mark.parametrize("T,H", [(50, 4096), (51, 256), (51, 512)])
def test_consumer_alone_matches_oracle(T, H):
    """The consumer on its own.  Without a post-norm it is compared with the
    oracle directly.  With one, the post-normed y (within 1 ulp) is read back
    through a zero residual, the oracle checks y and the consumer applied to
    the GPU's y, and the one-call result must equal the two-call one.  (At
    hidden 256 four tokens share a wave, at 512 two; 51 leaves the last
    wave three and one.)"""
    rng = np.random.Generator(np.random.PCG64(90 + H))
    x = wl.normal_bf16(rng, (T, H + 128))
    x[:, H:] = 0x7FC0
    res = wl.normal_bf16(rng, (T, H))
    pw = wl.normal_bf16(rng, (H,), mean=1.0, std=0.05)
    nw = wl.normal_bf16(rng, (H,), mean=1.0, std=0.1)
    xd, resd, pwd, nwd = dev_bf16(x)[:, :H], dev_bf16(res), dev_bf16(pw), dev_bf16(nw)
    # no post-norm
    h, n = mf.beam_norm_residual_norm(xd, resd, None, None, nwd, 1e-5, None)
    sync()
    wh, wn = oracle.beam_norm_residual_norm(x, res, None, None, nw, 1e-5, None)
    assert_bits_equal(host_bits(h), wh, "consumer hidden")
    assert_within_ulp(host_bits(n), wn, 1, NORM_MIN_EXACT, "consumer normalized")
    # with a post-norm
    zero = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    y, _ = mf.beam_norm_residual_norm(xd, zero, pwd, 1e-6, None, None, None)
    h1, n1 = mf.beam_norm_residual_norm(xd, resd, pwd, 1e-6, nwd, 1e-5, (0.25, 1.0))
    h2, n2 = mf.beam_norm_residual_norm(y, resd, None, None, nwd, 1e-5, (0.25, 1.0))
    sync()
    wy, _ = oracle.beam_norm_residual_norm(x, np.zeros((T, H), np.uint16), pw, 1e-6)
    assert_within_ulp(host_bits(y), wy, 1, NORM_MIN_EXACT, "consumer post-norm")
    assert_bits_equal(host_bits(h1), host_bits(h2), "one call vs two calls, hidden")
    assert_bits_equal(host_bits(n1), host_bits(n2), "one call vs two calls, normalized")
    ch, cn = oracle.beam_norm_residual_norm(host_bits(y), res, None, None, nw, 1e-5, (0.25, 1.0))
    assert_bits_equal(host_bits(h1), ch, "consumer hidden after post-norm")
    assert_within_ulp(host_bits(n1), cn, 1, NORM_MIN_EXACT, "consumer normalized after post-norm")


# ------------------------------------------------------------ edge cases ----

# 585 and 2048 tokens run in one round at 3 and 8 workgroups per CU (a
# 256-CU device), 2049 at the usual residency.
@pytest.mark.parametrize("T", [1, 7, 8, 9, 13, 257, 585, 2048, 2049])
def test_ragged_token_counts(T):
    c = wl.tiny(num_tokens=T, num_rows=8 * T + 3, invalid_frac=0.05, poison=True,
                nan_rows_beyond=2)
    d = IndexMapOnDevice(c)
    assert_within_ulp(gpu_rmsnorm(d), oracle_rmsnorm(c), 1, NORM_MIN_EXACT, f"T={T}")
    assert_bits_equal(gpu_finalize(d), oracle_finalize(c), f"T={T}")


# Index-map calls of a few hundred to two thousand tokens take the one-round
# residency (all tokens resident at once, up to 8 workgroups per CU on a
# 256-CU device) in every kernel kind: compile-time top-k 16 (5 per CU),
# run-time top-k sized for 12 slots (4 per CU), for 8 slots at two vectors
# per thread (6 per CU), the rolling window at hidden 7168 (3 per CU asked,
# registers hold 2), and tiny rows whose cap already holds them (16 per CU).
@pytest.mark.parametrize("H,K,T", [(2048, 16, 1170), (2048, 12, 1000), (4096, 5, 1300),
                                   (7168, 32, 585), (256, 1, 4000)])
def test_one_round_residency_shapes(H, K, T):
    c = wl.make_index_map_case(7000 + H + K, num_tokens=T, hidden=H, top_k=K,
                               num_rows=T * K + 7, row_stride=H + 8, weights_dtype="fp32",
                               invalid_frac=0.05, poison=True, nan_rows_beyond=2)
    d = IndexMapOnDevice(c)
    assert_within_ulp(gpu_rmsnorm(d), oracle_rmsnorm(c), 1, NORM_MIN_EXACT, f"H={H} K={K} T={T}")
    assert_bits_equal(gpu_finalize(d), oracle_finalize(c), f"H={H} K={K} T={T}")


# Hidden 256 at top-k up to 7: several tokens per wave (four at top-k 1, two
# at top-k 2-7), each lane group with its own slots, masking and norm; token
# counts that are not a multiple leave the last wave partly empty.  Top-k 8
# and 13 run one token per workgroup beside them.
@pytest.mark.parametrize("T", [1, 2, 3, 4, 6, 31, 2049])
def test_several_tokens_per_wave_at_hidden_256(T):
    for K, wdt in ((1, "bf16"), (2, "fp32"), (3, "fp32"), (4, "bf16"), (6, "fp32"), (7, "bf16"),
                   (8, "fp32"), (13, "bf16")):
        c = wl.make_index_map_case(8000 + T + K, num_tokens=T, hidden=256, top_k=K,
                                   num_rows=T * K + 9, row_stride=264, weights_dtype=wdt,
                                   invalid_frac=0.1, poison=True, nan_rows_beyond=2)
        d = IndexMapOnDevice(c)
        what = f"T={T} K={K} {wdt}"
        assert_bits_equal(gpu_finalize(d), oracle_finalize(c), what)
        for wbn in (False, True):
            assert_within_ulp(gpu_rmsnorm(d, weight_before_norm=wbn),
                              oracle_rmsnorm(c, weight_before_norm=wbn), 1, NORM_MIN_EXACT,
                              f"{what} wbn={wbn}")
    for K, norm in ((1, True), (2, False), (3, False), (4, True), (5, False), (7, True),
                    (16, True)):
        b = wl.make_token_major_case(8100 + T + K, capacity=T + 2, top_k=K, hidden=256,
                                     live_tokens=T, routed_scale=1.5,
                                     post_eps=1e-6 if norm else None,
                                     post_weight_std=0.05 if norm else None, poison_dead=True)
        bd = TokenMajorOnDevice(b)
        got, want = gpu_beam(bd), oracle_beam(b)
        if norm:
            assert_within_ulp(got, want, 1, NORM_MIN_EXACT, f"token major T={T} K={K}")
        else:
            assert_bits_equal(got, want, f"token major T={T} K={K}")


# Hidden 512 at top-k 1: two tokens per wave (32 lanes of two vectors
# each); top-k 2 runs one token per wave beside it.
@pytest.mark.parametrize("T", [1, 2, 3, 31, 2049])
def test_two_tokens_per_wave_at_hidden_512(T):
    for K, wdt in ((1, "bf16"), (1, "fp32"), (2, "fp32")):
        c = wl.make_index_map_case(8200 + T + K, num_tokens=T, hidden=512, top_k=K,
                                   num_rows=T * K + 9, row_stride=520, weights_dtype=wdt,
                                   invalid_frac=0.1, poison=True, nan_rows_beyond=2)
        d = IndexMapOnDevice(c)
        what = f"H=512 T={T} K={K} {wdt}"
        assert_bits_equal(gpu_finalize(d), oracle_finalize(c), what)
        for wbn in (False, True):
            assert_within_ulp(gpu_rmsnorm(d, weight_before_norm=wbn),
                              oracle_rmsnorm(c, weight_before_norm=wbn), 1, NORM_MIN_EXACT,
                              f"{what} wbn={wbn}")
    for norm in (False, True):
        b = wl.make_token_major_case(8300 + T, capacity=T + 2, top_k=1, hidden=512,
                                     live_tokens=T, routed_scale=1.5,
                                     post_eps=1e-6 if norm else None,
                                     post_weight_std=0.05 if norm else None, poison_dead=True)
        bd = TokenMajorOnDevice(b)
        got, want = gpu_beam(bd), oracle_beam(b)
        if norm:
            assert_within_ulp(got, want, 1, NORM_MIN_EXACT, f"token major H=512 T={T}")
        else:
            assert_bits_equal(got, want, f"token major H=512 T={T}")


def test_all_invalid_tokens_and_empty_row_matrix():
    c = wl.tiny(num_tokens=12, num_rows=96)
    c.idx[3, :] = -1
    c.idx[7, :] = 9999
    d = IndexMapOnDevice(c)
    got_n, got_f = gpu_rmsnorm(d), gpu_finalize(d)
    assert_within_ulp(got_n, oracle_rmsnorm(c), 1, NORM_MIN_EXACT, "all-invalid rmsnorm")
    assert_bits_equal(got_f, oracle_finalize(c), "all-invalid finalize")
    for t in (3, 7):
        assert np.all((got_n[t] & 0x7FFF) == 0) and np.all((got_f[t] & 0x7FFF) == 0)
    # no rows at all: every index is out of range
    empty = torch.empty((0, 4096), dtype=torch.bfloat16, device="cuda")
    out = d.new_output()
    mf.moe_finalize(empty, d.weights, d.idx, out)
    out2 = d.new_output()
    mf.moe_finalize_rmsnorm(empty, d.weights, d.idx, d.norm_weight, out2, eps=1e-6,
                            gain_center=1.0, weight_before_norm=False)
    sync()
    assert np.all((host_bits(out) & 0x7FFF) == 0)
    assert np.all((host_bits(out2) & 0x7FFF) == 0)


def test_zero_rows_launch_nothing():
    c = wl.tiny(num_tokens=4, num_rows=32)
    d = IndexMapOnDevice(c)
    out = d.new_output(0x1234)
    idx0 = d.idx[:0]
    w0 = d.weights[:0]
    mf.moe_finalize(d.gemm2, w0, idx0, out[:0])
    mf.moe_finalize_rmsnorm(d.gemm2, w0, idx0, d.norm_weight, out[:0], eps=1e-6,
                            gain_center=1.0, weight_before_norm=False)
    b = TokenMajorOnDevice(wl.make_token_major_case(5, capacity=4, top_k=2, hidden=256,
                                                    live_tokens=0))
    bout = b.new_output(0)
    mf.beam_moe_finalize(b.expert_outputs, b.weights, bout)
    sync()
    assert np.all(host_bits(out) == 0x1234)


def test_row_offsets_beyond_2_gib():
    """Rows whose byte offset exceeds 2^31 (70000 rows x 32 KiB stride,
    2.3 GB): the gather addresses them with 64-bit offsets.  The oracle gets
    the same rows compacted and the index map remapped accordingly."""
    R, S, H, T, K = 70000, 16384, 4096, 24, 8
    rng = np.random.Generator(np.random.PCG64(123))
    picked = np.sort(rng.choice(np.arange(R - 4000, R), size=T * K, replace=False))
    assert int(picked[0]) * S * 2 > 2 ** 31
    rows = wl.normal_bf16(rng, (T * K, H))
    order = rng.permutation(T * K)
    idx_small = order.reshape(T, K).astype(np.int32)            # into the compact rows
    idx_big = picked[order].reshape(T, K).astype(np.int32)      # into the big matrix
    idx_small[0, 3] = -1
    idx_big[0, 3] = -1
    w = wl.softmax_rows(rng.standard_normal((T, K)))
    nw = wl.normal_bf16(rng, (H,), std=0.1)
    big = torch.full((R, S), float("nan"), dtype=torch.bfloat16, device="cuda")
    big[torch.from_numpy(picked).cuda(), :H] = dev_bf16(rows)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    mf.moe_finalize_rmsnorm(big, torch.from_numpy(w).cuda(), torch.from_numpy(idx_big).cuda(),
                            dev_bf16(nw), out, eps=1e-6, gain_center=1.0,
                            weight_before_norm=False)
    out2 = torch.empty_like(out)
    mf.moe_finalize(big, torch.from_numpy(w).cuda(), torch.from_numpy(idx_big).cuda(), out2)
    sync()
    want = oracle.moe_finalize_rmsnorm(rows, w, idx_small, nw, eps=1e-6, gain_center=1.0,
                                       weight_before_norm=False)
    assert_within_ulp(host_bits(out), want, 1, NORM_MIN_EXACT, "rows past 2 GiB, norm")
    assert_bits_equal(host_bits(out2), oracle.moe_finalize(rows, w, idx_small, H),
                      "rows past 2 GiB, finalize")
    del big


def test_live_equals_capacity_and_partial_live():
    c = wl.make_token_major_case(77, capacity=40, top_k=8, hidden=7168, live_tokens=40,
                                 routed_scale=2.5)
    d = TokenMajorOnDevice(c)
    assert_bits_equal(gpu_beam(d), oracle_beam(c), "live == capacity")
    assert_bits_equal(gpu_beam(d, 17), oracle_beam(c, 17), "live 17")


def test_extreme_values_propagate_like_the_oracle():
    """Overflow to infinity, NaN in a valid row and huge weights behave as the
    oracle's IEEE arithmetic says (compared by NaN-ness and bits).  The norm
    is compared only where its FP32 sum of squares cannot overflow: the
    oracle keeps that sum in binary64."""
    c = wl.tiny(num_tokens=8, num_rows=64, invalid_frac=0.0)
    g = c.gemm2_storage
    g[c.idx[0, 0]] = wl.to_bf16_bits(np.full(4096, 3e38, np.float32))
    g[c.idx[0, 1]] = wl.to_bf16_bits(np.full(4096, 3e38, np.float32))
    c.expert_weights[0, :2] = 1.0                     # 6e38 -> +inf
    g[c.idx[1, 3], 100:200] = 0x7FC0                  # NaN in a valid row
    c.expert_weights[2, 5] = np.float32(1e30)         # large finite weight
    d = IndexMapOnDevice(c)
    assert_bits_equal(gpu_finalize(d), oracle_finalize(c), "extreme finalize")
    keep = [t for t in range(8) if t != 2]
    assert_within_ulp(gpu_rmsnorm(d)[keep], oracle_rmsnorm(c)[keep], 1, NORM_MIN_EXACT,
                      "extreme rmsnorm (NaN/inf rows)")


@pytest.mark.parametrize("post,post_w,nxt,next_w,scales", [
    (True, True, True, True, (0.5, 2.0)), (False, False, True, False, None),
    (True, False, False, False, (1.0, -1.0)),
])
def test_strategy_unfused_equals_fused(post, post_w, nxt, next_w, scales):
    """The page's strategy keyword: "unfused" (finalize into a BF16
    intermediate, then the consumer) and "fused" give the default fused
    call's outputs bit for bit."""
    c, res, nw, next_eps, scales = residual_case(77, 40, 6, 2048, 33, post, post_w, nxt, next_w,
                                                 scales, 1.25)
    d = TokenMajorOnDevice(c)
    resd = dev_bf16(res)
    nwd = None if nw is None else dev_bf16(nw)
    outs = {}
    for strategy in (None, "fused", "unfused"):
        outs[strategy] = mf.beam_moe_finalize_norm_residual_norm(
            d.expert_outputs, d.weights, resd, d.post_weight, c.post_eps, nwd, next_eps, scales,
            c.routed_scale, strategy=strategy)
    sync()
    h0, n0 = outs[None]
    for strategy in ("fused", "unfused"):
        h, n = outs[strategy]
        assert_bits_equal(host_bits(h), host_bits(h0), f"{strategy} hidden")
        assert (n is None) == (n0 is None)
        if n is not None:
            assert_bits_equal(host_bits(n), host_bits(n0), f"{strategy} normalized")


def test_hardware_bf16_rounding_matches_round_to_nearest_even():
    """K = 1 and rows of 1.0 make the output bf16(weight): the packed convert
    is checked on ties, subnormals, overflow and NaN against the oracle's
    rounding (pinned to torch's cast)."""
    x = _f32_probe_values(np.random.Generator(np.random.PCG64(31)))
    n = x.size
    H = 256
    e = np.full((n, 1, H), 0x3F80, np.uint16)
    case_ = wl.TokenMajorCase(e, x.reshape(n, 1).astype(np.float32), n, 1.0, None, None)
    d = TokenMajorOnDevice(case_)
    got = gpu_beam(d)
    want = oracle_beam(case_)
    assert_bits_equal(got, want, "beam bf16(w)")
    rows = np.full((1, H), 0x3F80, np.uint16)
    im = wl.IndexMapCase(rows, 1, H, x.reshape(n, 1).astype(np.float32),
                         np.zeros((n, 1), np.int32), np.zeros(H, np.uint16), 1e-6, 0.0, False)
    assert_bits_equal(gpu_finalize(IndexMapOnDevice(im)), oracle_finalize(im), "finalize bf16(w)")


def test_graph_capture_and_replay():
    """The entry points allocate, synchronise and memset nothing, so they can
    be captured in a HIP graph: every replay (with eager work and
    synchronisation between replays) must equal the eager launch."""
    c = wl.tiny(num_tokens=64, num_rows=512, invalid_frac=0.05)
    d = IndexMapOnDevice(c)
    b = wl.make_token_major_case(9, capacity=48, top_k=8, hidden=2048, live_tokens=40,
                                 routed_scale=1.5, post_eps=1e-6, post_weight_std=0.05)
    bd = TokenMajorOnDevice(b)
    rng = np.random.Generator(np.random.PCG64(10))
    res = dev_bf16(wl.normal_bf16(rng, (40, 2048)))
    nw = dev_bf16(wl.normal_bf16(rng, (2048,), mean=1.0, std=0.1))
    out = d.new_output()
    h = torch.empty((40, 2048), dtype=torch.bfloat16, device="cuda")
    n = torch.empty_like(h)

    def launch():
        mf.moe_finalize_rmsnorm(d.gemm2, d.weights, d.idx, d.norm_weight, out, eps=c.eps,
                                gain_center=c.gain_center, weight_before_norm=False)
        mf.beam_moe_finalize_norm_residual_norm(bd.expert_outputs, bd.weights, res,
                                                bd.post_weight, b.post_eps, nw, 1e-6, None,
                                                b.routed_scale, hidden_out=h, normalized_out=n)

    launch()                       # eager (also warms every lazily queried attribute)
    sync()
    want = (host_bits(out), host_bits(h), host_bits(n))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        launch()
    torch.cuda.current_stream().wait_stream(s)
    sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    for rep in range(3):
        out.fill_(0.0)
        h.fill_(0.0)
        n.fill_(0.0)
        sync()
        g.replay()
        sync()
        got = (host_bits(out), host_bits(h), host_bits(n))
        for name, x, y in zip(("rmsnorm", "hidden", "normalized"), got, want):
            assert_bits_equal(x, y, f"graph replay {rep} {name}")


def test_concurrent_streams_match_serial_results():
    """Different entry points running at the same time on two streams give
    the results they give alone (no shared state in the library)."""
    c = wl.tiny(num_tokens=512, num_rows=4096, invalid_frac=0.02)
    d = IndexMapOnDevice(c)
    b = wl.make_token_major_case(12, capacity=600, top_k=16, hidden=2048, live_tokens=600,
                                 routed_scale=1.0, post_eps=1e-6, post_weight_std=0.05)
    bd = TokenMajorOnDevice(b)
    o1, o2 = d.new_output(), bd.new_output()
    mf.moe_finalize_rmsnorm(d.gemm2, d.weights, d.idx, d.norm_weight, o1, eps=c.eps,
                            gain_center=c.gain_center, weight_before_norm=False)
    mf.beam_moe_finalize(bd.expert_outputs, bd.weights, o2, 1.0, bd.post_weight, 1e-6)
    sync()
    want1, want2 = host_bits(o1), host_bits(o2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(4):
        p1, p2 = d.new_output(), bd.new_output()
        sync()
        with torch.cuda.stream(s1):
            mf.moe_finalize_rmsnorm(d.gemm2, d.weights, d.idx, d.norm_weight, p1, eps=c.eps,
                                    gain_center=c.gain_center, weight_before_norm=False)
        with torch.cuda.stream(s2):
            mf.beam_moe_finalize(bd.expert_outputs, bd.weights, p2, 1.0, bd.post_weight, 1e-6)
        outs.append((p1, p2))
    sync()
    for p1, p2 in outs:
        assert_bits_equal(host_bits(p1), want1, "stream 1")
        assert_bits_equal(host_bits(p2), want2, "stream 2")


def test_runs_on_the_given_stream():
    c = wl.tiny(num_tokens=32, num_rows=256)
    d = IndexMapOnDevice(c)
    s = torch.cuda.Stream()
    out = d.new_output()
    torch.cuda.current_stream().synchronize()
    with torch.cuda.stream(s):
        mf.moe_finalize_rmsnorm(d.gemm2, d.weights, d.idx, d.norm_weight, out, eps=c.eps,
                                gain_center=c.gain_center, weight_before_norm=False)
    s.synchronize()
    assert_within_ulp(host_bits(out), oracle_rmsnorm(c), 1, NORM_MIN_EXACT, "side stream")


def test_host_threads_call_concurrently():
    """The library keeps no shared mutable state beyond a per-device cache of
    LDS limits: host threads launching on their own streams at the same time
    get the results of serial calls."""
    import threading
    c = wl.tiny(num_tokens=300, num_rows=2400, invalid_frac=0.03)
    d = IndexMapOnDevice(c)
    want = gpu_rmsnorm(d)
    outs, errors = [], []

    def worker(seed):
        try:
            s = torch.cuda.Stream()
            mine = [d.new_output() for _ in range(8)]
            sync()
            with torch.cuda.stream(s):
                for o in mine:
                    mf.moe_finalize_rmsnorm(d.gemm2, d.weights, d.idx, d.norm_weight, o,
                                            eps=c.eps, gain_center=c.gain_center,
                                            weight_before_norm=False)
            s.synchronize()
            outs.extend(mine)
        except Exception as e:   # reported on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    assert len(outs) == 32
    for o in outs:
        assert_bits_equal(host_bits(o), want, "threaded call")


def test_output_offsets_beyond_4_gib_sampled():
    """2.2 M tokens of hidden 1024 (4.5 GB of output, its second half past
    2^32 bytes) gathering from 65536 shared rows, with 1.5 % of the indices
    negative: a grid of millions of workgroups and 64-bit token and output
    offsets.  Sampled tokens, spread over the whole
    range and including the last, are compared with the oracle."""
    T, H, K, R = 2_200_000, 1024, 2, 65536
    assert T * H * 2 > 2 ** 32
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    rows = torch.randn((R, H), generator=gen, device="cuda").to(torch.bfloat16)
    idx = torch.randint(-R // 64, R, (T, K), generator=gen, device="cuda", dtype=torch.int32)
    w = torch.softmax(torch.randn((T, K), generator=gen, device="cuda"), dim=1)
    nw = (1.0 + 0.1 * torch.randn(H, generator=gen, device="cuda")).to(torch.bfloat16)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    mf.moe_finalize_rmsnorm(rows, w, idx, nw, out, eps=1e-6, gain_center=0.0,
                            weight_before_norm=True)
    sync()
    rng = np.random.Generator(np.random.PCG64(78))
    pick = np.unique(np.concatenate([rng.integers(0, T, 2000), [0, T - 1, 2 ** 21 + 5]]))
    pick_t = torch.from_numpy(pick).cuda()
    got = host_bits(out[pick_t])
    want = oracle.moe_finalize_rmsnorm(host_bits(rows), w[pick_t].cpu().numpy(),
                                       idx[pick_t].cpu().numpy(), host_bits(nw), eps=1e-6,
                                       gain_center=0.0, weight_before_norm=True)
    assert_within_ulp(got, want, 1, NORM_MIN_EXACT, "sampled tokens past 4 GiB of output")
    del out, rows
    torch.cuda.empty_cache()


def test_token_major_offsets_beyond_4_gib_sampled():
    """Token-major rows of 300 000 tokens x top-k 8 x hidden 1024 (4.9 GB):
    the rows of the later tokens start past 2^32 bytes.  Sampled tokens are
    compared with the oracle on their own rows."""
    C, K, H = 300_000, 8, 1024
    assert C * K * H * 2 > 2 ** 32
    gen = torch.Generator(device="cuda")
    gen.manual_seed(79)
    e = torch.empty((C, K, H), dtype=torch.bfloat16, device="cuda")
    for s in range(0, C, 50_000):        # in slices: no 10 GB FP32 temporary
        e[s:s + 50_000] = torch.randn((min(50_000, C - s), K, H), generator=gen,
                                      device="cuda").to(torch.bfloat16)
    w = torch.softmax(torch.randn((C, K), generator=gen, device="cuda"), dim=1)
    pw = (1.0 + 0.05 * torch.randn(H, generator=gen, device="cuda")).to(torch.bfloat16)
    out = torch.empty((C, H), dtype=torch.bfloat16, device="cuda")
    mf.beam_moe_finalize(e, w, out, 1.5, pw, 1e-6)
    sync()
    rng = np.random.Generator(np.random.PCG64(80))
    pick = np.unique(np.concatenate([rng.integers(0, C, 1000), [0, C - 1]]))
    pick_t = torch.from_numpy(pick).cuda()
    got = host_bits(out[pick_t])
    want = oracle.beam_moe_finalize(host_bits(e[pick_t]), w[pick_t].cpu().numpy(), len(pick),
                                    1.5, host_bits(pw), 1e-6)
    assert_within_ulp(got, want, 1, NORM_MIN_EXACT, "sampled token-major rows past 4 GiB")
    del e, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("H", [1024, 256, 512])
def test_negative_zero_passes_through_direct_rows(H):
    """Rows read directly (the standalone norm and the residual consumer)
    keep -0: the sum starts from -0, so fma(1, -0, -0) stays -0 where a +0
    start would turn it into +0.  Elements whose oracle value is a zero must
    match it bit for bit, sign included (the ulp comparison counts +0 and -0
    as equal); the rest within 1 ulp.  Hidden 256 runs four tokens per wave
    and 512 two (9 tokens: the last wave holds one)."""
    rng = np.random.Generator(np.random.PCG64(97))
    T = 9
    x = wl.normal_bf16(rng, (T, H))
    x[:, ::5] = 0x8000                               # -0 in a fifth of the columns
    x[:, 1::7] = 0x0000
    res = np.full((T, H), 0x8000, np.uint16)         # residual -0 everywhere
    res[:, 3::4] = wl.normal_bf16(rng, (T, len(range(3, H, 4))))
    nw = wl.normal_bf16(rng, (H,), mean=0.0, std=1.0)  # mixed signs: -0 * g < 0 gives +0
    xd, resd, nwd = dev_bf16(x), dev_bf16(res), dev_bf16(nw)

    def check(got, want, what):
        zero = (want & 0x7FFF) == 0
        assert zero.any()
        assert np.array_equal(got[zero], want[zero]), f"{what}: signed zeros differ"
        assert_within_ulp(got, want, 1, NORM_MIN_EXACT, what)

    for wbn in (False, True):
        out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        mf.mf_rmsnorm(xd, nwd, out, eps=1e-6, gain_center=0.0, weight_before_norm=wbn)
        sync()
        want = oracle.rmsnorm(x, nw, eps=1e-6, gain_center=0.0, weight_before_norm=wbn)
        check(host_bits(out), want, f"mf_rmsnorm wbn={wbn}")
    h, n = mf.beam_norm_residual_norm(xd, resd, None, None, nwd, 1e-6, None)
    sync()
    wh, wn = oracle.beam_norm_residual_norm(x, res, None, None, nw, 1e-6, None)
    assert np.array_equal(host_bits(h), wh), "hidden = x + residual differs (signed zeros)"
    check(host_bits(n), wn, "normalized")


def _split_sample(T, boundary, seed):
    """Tokens to compare on a call split into launches: both sides of the
    first launch boundary, the first and last tokens, and a random spread."""
    rng = np.random.Generator(np.random.PCG64(seed))
    near = np.arange(boundary - 64, boundary + 64)
    return np.unique(np.concatenate([np.arange(64), near, np.arange(T - 64, T),
                                     rng.integers(0, T, 1000)]))


# (hidden, top-k, threads per workgroup, tokens per workgroup): hidden 256
# holds four tokens per wave at top-k 1 and two at top-k 2, hidden 512 two at
# top-k 1, hidden 768 leaves half a wave idle.
@pytest.mark.parametrize("H,K,team,tpw", [(256, 1, 64, 4), (256, 2, 64, 2), (512, 1, 64, 2),
                                          (768, 1, 128, 1), (4096, 8, 512, 1)])
def test_index_map_split_into_launches_sampled(H, K, team, tpw):
    """A token count whose grid exceeds the 2^31 work-items one launch may
    span (teams of `team` threads, `tpw` tokens each): the call runs as
    several launches, each from its own first token; the remainder of 3001
    leaves the last multi-token wave one token.  Tokens on both sides of the
    first launch boundary, at both ends and spread over the range are
    compared with the oracle (top-k 1 without a norm: bit-exact; otherwise
    with the norm: within 1 ulp)."""
    per_launch = 2 ** 31 // team * tpw
    T, R = per_launch + 3001, 4096
    gen = torch.Generator(device="cuda")
    gen.manual_seed(90 + K)
    rows = torch.randn((R, H), generator=gen, device="cuda").to(torch.bfloat16)
    idx = torch.randint(-R // 64, R, (T, K), generator=gen, device="cuda", dtype=torch.int32)
    w = torch.softmax(torch.randn((T, K), generator=gen, device="cuda"), dim=1)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    pick = _split_sample(T, per_launch, 91 + K)
    pick_t = torch.from_numpy(pick).cuda()
    if K == 1:
        mf.moe_finalize(rows, w, idx, out)
        sync()
        want = oracle.moe_finalize(host_bits(rows), w[pick_t].cpu().numpy(),
                                   idx[pick_t].cpu().numpy(), H)
        assert_bits_equal(host_bits(out[pick_t]), want, "tokens across the launch split")
    else:
        nw = (0.1 * torch.randn(H, generator=gen, device="cuda")).to(torch.bfloat16)
        mf.moe_finalize_rmsnorm(rows, w, idx, nw, out, eps=1e-6, gain_center=1.0,
                                weight_before_norm=False)
        sync()
        want = oracle.moe_finalize_rmsnorm(host_bits(rows), w[pick_t].cpu().numpy(),
                                           idx[pick_t].cpu().numpy(), host_bits(nw), eps=1e-6,
                                           gain_center=1.0, weight_before_norm=False)
        assert_within_ulp(host_bits(out[pick_t]), want, 1, NORM_MIN_EXACT,
                          "tokens across the launch split")
    del out, idx, w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("H,team,tpw", [(256, 64, 4), (768, 128, 1)])
def test_token_major_split_into_launches_sampled(H, team, tpw):
    """Token-major rows at top-k 1 for one launch's tokens plus 3001 (hidden
    256: four tokens per wave, 2^27 + 3001 live tokens, 69 GB of rows; hidden
    768: 2^24 + 3001, 26 GB): two launches.  Sampled tokens around the
    boundary and across the range are compared with the oracle bit for bit
    (no norm, routed_scale 1.25)."""
    per_launch = 2 ** 31 // team * tpw
    C = per_launch + 3001
    gen = torch.Generator(device="cuda")
    gen.manual_seed(95)
    e = torch.empty((C, 1, H), dtype=torch.bfloat16, device="cuda")
    for s in range(0, C, 1 << 24):
        n = min(1 << 24, C - s)
        e[s:s + n] = torch.randn((n, 1, H), generator=gen, device="cuda").to(torch.bfloat16)
    w = torch.rand((C, 1), generator=gen, device="cuda") + 0.5
    out = torch.empty((C, H), dtype=torch.bfloat16, device="cuda")
    mf.beam_moe_finalize(e, w, out, 1.25)
    sync()
    pick = _split_sample(C, per_launch, 96)
    pick_t = torch.from_numpy(pick).cuda()
    want = oracle.beam_moe_finalize(host_bits(e[pick_t]), w[pick_t].cpu().numpy(), len(pick),
                                    1.25)
    assert_bits_equal(host_bits(out[pick_t]), want, "token-major tokens across the launch split")
    del e, out
    torch.cuda.empty_cache()


def test_repeated_launches_are_deterministic():
    """2000 back-to-back prefill-shaped launches into four rotating outputs:
    every output is bit-identical to the first launch's (the result depends
    on nothing but the inputs: no atomics, no order-dependent reduction)."""
    c = case("prefill", INDEX_CONFIGS["prefill"])
    d = IndexMapOnDevice(c)
    first = gpu_rmsnorm(d)
    outs = [d.new_output() for _ in range(4)]
    for i in range(2000):
        mf.moe_finalize_rmsnorm(d.gemm2, d.weights, d.idx, d.norm_weight, outs[i % 4],
                                eps=c.eps, gain_center=c.gain_center,
                                weight_before_norm=c.weight_before_norm)
    sync()
    for j, o in enumerate(outs):
        assert_bits_equal(host_bits(o), first, f"output {j} after 2000 launches")
