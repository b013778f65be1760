"""Property tests of the CPU oracle over random small shapes (hypothesis).

Each property follows from the method's definition on the finalize pages
(FlashInfer "flashinfer.comm.tp_moe_finalize_rmsnorm", description and
Parameters; vLLM "vllm.models.beam.nvidia.moe_finalize", beam_moe_finalize),
independently of how the oracle computes it.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import workloads as wl
from oracle_pins import assert_bits_equal, assert_within_ulp, f32_equal_pm0

SETTINGS = settings(max_examples=40, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def index_cases(draw):
    H = 256 * draw(st.integers(1, 3))
    K = draw(st.integers(1, 9))
    T = draw(st.integers(1, 6))
    R = draw(st.integers(1, 40))
    pad = 8 * draw(st.integers(0, 3))
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.Generator(np.random.PCG64(seed))
    g = wl.normal_bf16(rng, (R, H + pad))
    idx = rng.integers(-3, R + 3, size=(T, K)).astype(np.int32)
    w = rng.standard_normal((T, K)).astype(np.float32)
    return g, R, H, idx, w, rng


@SETTINGS
@given(index_cases())
def test_invalid_slot_equals_zero_weight(case):
    """An out-of-range index contributes exactly what a valid index with
    weight 0 contributes (fma(0, x, acc) == acc for finite x)."""
    g, R, H, idx, w, rng = case
    bad = (idx < 0) | (idx >= R)
    idx2 = np.where(bad, 0, idx).astype(np.int32)
    w2 = np.where(bad, np.float32(0), w).astype(np.float32)
    a = oracle.routed_sum(g, w, idx, H, num_rows=R)
    b = oracle.routed_sum(g, w2, idx2, H, num_rows=R)
    assert f32_equal_pm0(a, b)


@SETTINGS
@given(index_cases())
def test_power_of_two_weight_scaling_commutes(case):
    """Scaling every weight by 2^k scales the FP32 sum by exactly 2^k (no
    overflow or underflow at these magnitudes)."""
    g, R, H, idx, w, rng = case
    a = oracle.routed_sum(g, w, idx, H, num_rows=R)
    b = oracle.routed_sum(g, (w * np.float32(4.0)).astype(np.float32), idx, H, num_rows=R)
    assert f32_equal_pm0(b, a * np.float32(4.0))


@SETTINGS
@given(index_cases())
def test_norm_output_rms(case):
    """With the weight before the norm and a negligible eps, the output RMS is
    1 up to BF16 rounding for any token whose sum is not tiny."""
    g, R, H, idx, w, rng = case
    nw = wl.normal_bf16(rng, (H,), mean=1.0, std=0.2)
    out = oracle.moe_finalize_rmsnorm(g, w, idx, nw, eps=1e-30, gain_center=0.0,
                                      weight_before_norm=True, num_rows=R)
    acc = oracle.routed_sum(g, w, idx, H, num_rows=R)
    y = wl.bf16_bits_to_f32(out).astype(np.float64)
    for t in range(idx.shape[0]):
        if np.abs(acc[t]).max() > 1e-2:
            rms = np.sqrt(np.mean(y[t] ** 2))
            assert abs(rms - 1.0) < 1e-2


@SETTINGS
@given(st.integers(0, 2**31 - 1), st.integers(1, 5), st.integers(1, 3),
       st.sampled_from([1.0, 2.5, 0.5, 3.0]))
def test_beam_token_order_independence(seed, K, n, scale):
    """Each token's output depends only on its own rows and weights: finalizing
    a permutation of the tokens permutes the outputs."""
    H = 256 * n
    rng = np.random.Generator(np.random.PCG64(seed))
    C = 6
    e = wl.normal_bf16(rng, (C, K, H))
    w = rng.random((C, K)).astype(np.float32)
    perm = rng.permutation(C)
    a = oracle.beam_moe_finalize(e, w, C, scale)
    b = oracle.beam_moe_finalize(np.ascontiguousarray(e[perm]), w[perm], C, scale)
    assert_bits_equal(b, a[perm], "token permutation")


@SETTINGS
@given(st.integers(0, 2**31 - 1), st.integers(1, 3))
def test_post_norm_scale_invariance(seed, n):
    """The beam post-norm output does not change when routed_scale is a power
    of two (the scale is exact and cancels in the norm, eps negligible)."""
    H = 256 * n
    rng = np.random.Generator(np.random.PCG64(seed))
    e = wl.normal_bf16(rng, (4, 3, H))
    w = rng.random((4, 3)).astype(np.float32)
    pw = wl.normal_bf16(rng, (H,), mean=1.0, std=0.1)
    a = oracle.beam_moe_finalize(e, w, 4, 1.0, pw, 1e-12)
    b = oracle.beam_moe_finalize(e, w, 4, 4.0, pw, 1e-12)
    assert_within_ulp(a, b, 0, 1.0, "power-of-two routed_scale")
