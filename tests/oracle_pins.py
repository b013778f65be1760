"""Pins that tie the CPU oracle to facts other than itself.

Each ``pin_*`` takes an oracle module (the real ``oracle`` package, or a
deliberately broken copy built by the mutation test) and raises
AssertionError when the oracle disagrees with:

  - library routines: torch's CPU float32 -> bfloat16 cast and bfloat16 ->
    float32 widening, torch's rms_norm in float64;
  - brute force: nearest-value search over the full BF16 table, and exact
    rational arithmetic (fractions) for the FP32 fused multiply-add chain;
  - closed forms and invariants of the method.

Sources for what is pinned: FlashInfer page
"flashinfer.comm.tp_moe_finalize_rmsnorm" (description; Parameters eps,
gain_center, weight_before_norm) and vLLM page
"vllm.models.beam.nvidia.moe_finalize" (beam_moe_finalize docstring and
routed_scale / post_weight / post_eps parameters).
"""
from __future__ import annotations

import bisect
import math
from fractions import Fraction

import numpy as np
import torch

import workloads as wl

# ------------------------------------------------------------ BF16 helpers ---

_BF16_POS_BITS = np.arange(0, 0x7F81, dtype=np.uint32).astype(np.uint16)  # +0 .. +inf
_BF16_POS_VALS = wl.bf16_bits_to_f32(_BF16_POS_BITS).astype(np.float64)
_BF16_POS_VALS[-1] = 2.0 ** 128           # +inf competes as the next grid point
_BF16_VALS_LIST = list(_BF16_POS_VALS)


def torch_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """torch's CPU float32 -> bfloat16 cast, as uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def table_round_to_bf16(x) -> np.ndarray:
    """Nearest BF16 of binary64 values by search in the full BF16 table,
    ties to the even pattern; NaN -> quiet NaN."""
    x = np.atleast_1d(np.asarray(x, dtype=np.float64))
    a = np.abs(x)
    j = np.searchsorted(_BF16_POS_VALS, a, side="right") - 1
    j = np.clip(j, 0, len(_BF16_POS_VALS) - 2)
    lo = _BF16_POS_VALS[j]
    hi = _BF16_POS_VALS[j + 1]
    mid = (lo + hi) * 0.5                     # exact: both have <= 9 sig. bits
    lo_bits = _BF16_POS_BITS[j]
    up = (a > mid) | ((a == mid) & ((lo_bits & 1) == 1))
    bits = np.where(up, _BF16_POS_BITS[j + 1], lo_bits).astype(np.uint16)
    bits = np.where(a == np.inf, np.uint16(0x7F80), bits).astype(np.uint16)
    bits = np.where(np.signbit(x), bits | np.uint16(0x8000), bits).astype(np.uint16)
    bits = np.where(np.isnan(x), np.where(np.signbit(x), np.uint16(0xFFC0),
                                          np.uint16(0x7FC0)), bits)
    return bits.astype(np.uint16)


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in BF16 grid steps; +0 and -0 are equal; NaN vs NaN is 0 and
    NaN vs non-NaN is a huge distance."""
    a = np.asarray(a, dtype=np.uint16).astype(np.int64)
    b = np.asarray(b, dtype=np.uint16).astype(np.int64)

    def ordered(v):
        mag = v & 0x7FFF
        return np.where(v & 0x8000, -mag, mag)

    d = np.abs(ordered(a) - ordered(b))
    na = ((a & 0x7F80) == 0x7F80) & ((a & 0x7F) != 0)
    nb = ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    d = np.where(na | nb, np.where(na & nb, 0, 1 << 20), d)
    return d


def assert_bits_equal(got, want, what=""):
    d = bf16_ulp_distance(got, want)
    bad = np.flatnonzero(d.reshape(-1) != 0)
    assert bad.size == 0, (f"{what}: {bad.size} of {d.size} differ; first at flat "
                           f"{bad[0]}: got {np.asarray(got).reshape(-1)[bad[0]]:#06x} "
                           f"want {np.asarray(want).reshape(-1)[bad[0]]:#06x}")


def assert_within_ulp(got, want, max_ulp=1, min_exact=0.0, what=""):
    d = bf16_ulp_distance(got, want)
    worst = int(d.max()) if d.size else 0
    assert worst <= max_ulp, f"{what}: max ulp distance {worst} > {max_ulp}"
    if d.size:
        exact = float((d == 0).mean())
        assert exact >= min_exact, f"{what}: only {exact:.4f} bit-exact (< {min_exact})"


# ------------------------------------------------- exact FP32 FMA (Fraction) --

def nearest_f32(q: Fraction) -> np.float32:
    """Nearest binary32 to a rational, ties to even, by checking the
    neighbours of a nearby candidate."""
    c = np.float32(float(q))
    if not np.isfinite(c):
        c = np.float32(np.copysign(np.finfo(np.float32).max, float(q)))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best, best_key = None, None
    for v in cands:
        if not np.isfinite(v):
            continue
        dist = abs(Fraction(float(v)) - q)
        odd = int(np.array(v, dtype=np.float32).view(np.uint32)) & 1
        key = (dist, odd)
        if best_key is None or key < best_key:
            best, best_key = v, key
    return np.float32(best)


def exact_routed_sum(rows_bits: np.ndarray, num_rows: int, weights: np.ndarray,
                     idx: np.ndarray, hidden: int) -> np.ndarray:
    """Rational-arithmetic model of the FP32 routed reduction: per element, a
    chain over ascending slots of (w*x + acc) rounded once to binary32."""
    T, K = idx.shape
    w32 = weights if weights.dtype == np.float32 else wl.bf16_bits_to_f32(weights)
    out = np.zeros((T, hidden), dtype=np.float32)
    for t in range(T):
        for h in range(hidden):
            acc = np.float32(0.0)
            for k in range(K):
                i = int(idx[t, k])
                if not (0 <= i < num_rows):
                    continue
                x = Fraction(float(wl.bf16_bits_to_f32(rows_bits[i, h])))
                w = Fraction(float(w32[t, k]))
                acc = nearest_f32(w * x + Fraction(float(acc)))
            out[t, h] = acc
    return out


def f32_equal_pm0(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    same_bits = a.view(np.uint32) == b.view(np.uint32)
    both_zero = (a == 0) & (b == 0)
    return bool(np.all(same_bits | both_zero))


# ------------------------------------------------------------------ pins -----

def pin_bf16_widening(orc):
    """BF16 -> FP32 widening equals torch's for every pattern."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = np.array([orc.bf16_to_f32(int(b)) for b in bits], dtype=np.float32)
    nan_w = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan_w)
    assert np.array_equal(got[~nan_w].view(np.uint32), want[~nan_w].view(np.uint32))


def _f32_probe_values(rng) -> np.ndarray:
    ties = np.array([0x3F808000, 0x3F818000, 0x3F80C000, 0x3F807FFF, 0x3F808001,
                     0xBF808000, 0xBF818000, 0x7F7F8000, 0x7F7FFFFF, 0x7F7F7FFF,
                     0x00008000, 0x00018000, 0x00007FFF, 0x80008000, 0x007F8000,
                     0x00800000, 0x7F800000, 0xFF800000, 0x00000000, 0x80000000,
                     0x7FC00000, 0x7F800001, 0xFFC00001, 0x33800000, 0x3F7FFFFF],
                    dtype=np.uint32)
    rand = rng.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    near = rng.integers(0, 1 << 16, size=6000, dtype=np.uint64).astype(np.uint32) << 16
    near = near | rng.choice(np.array([0x8000, 0x7FFF, 0x8001, 0x0001, 0xFFFF],
                                      dtype=np.uint32), size=near.size)
    return np.concatenate([ties, rand, near]).view(np.float32)


def pin_rne_against_torch(orc):
    """FP32 -> BF16 rounding (ties, subnormals, overflow, NaN) equals torch's
    CPU cast, which rounds to nearest even."""
    rng = np.random.Generator(np.random.PCG64(11))
    x = _f32_probe_values(rng)
    want = torch_bf16_bits(x)
    got = np.array([orc.round_to_bf16(float(v)) for v in x], dtype=np.uint16)
    nan = np.isnan(x)
    assert np.all(((got[nan] & 0x7F80) == 0x7F80) & ((got[nan] & 0x7F) != 0))
    assert np.array_equal(got[~nan], want[~nan]), "BF16 rounding differs from torch"
    # the table search agrees with torch too, so it can stand in for binary64
    assert np.array_equal(table_round_to_bf16(x[~nan].astype(np.float64)), want[~nan])


def _f64_probe_values(rng) -> np.ndarray:
    # midpoints between neighbouring BF16 values, nudged by amounts that a
    # binary32 intermediate would erase (double rounding would go wrong here)
    b = rng.integers(1, 0x7F7F, size=3000).astype(np.uint16)
    lo = wl.bf16_bits_to_f32(b).astype(np.float64)
    hi = wl.bf16_bits_to_f32(b + 1).astype(np.float64)
    mid = 0.5 * (lo + hi)
    nudge = mid * np.ldexp(1.0, -40)
    vals = [mid, mid + nudge, mid - nudge, -mid, -(mid + nudge),
            rng.standard_normal(2000) * np.exp(rng.uniform(-100, 100, size=2000)),
            np.array([2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -140,
                      (2 - 2.0 ** -8) * 2.0 ** 127, (2 - 2.0 ** -8) * 2.0 ** 127 * (1 - 1e-15),
                      1e300, -1e300, 5e-324, 0.0, -0.0, np.inf, -np.inf])]
    return np.concatenate(vals)


def pin_rne_binary64_single_rounding(orc):
    """Binary64 -> BF16 rounds once (no binary32 intermediate): agrees with
    nearest-value search in the BF16 table, including nudged midpoints."""
    rng = np.random.Generator(np.random.PCG64(12))
    x = _f64_probe_values(rng)
    want = table_round_to_bf16(x)
    got = np.array([orc.round_to_bf16(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want), "binary64 -> BF16 rounding is wrong"
    # and a few of those cases by exact rational comparison
    for v in x[:40]:
        a = abs(Fraction(float(v)))
        j = bisect.bisect_right(_BF16_VALS_LIST, float(a)) - 1
        lo, hi = Fraction(_BF16_VALS_LIST[j]), Fraction(_BF16_VALS_LIST[j + 1])
        pick = j + 1 if (a - lo > hi - a or (a - lo == hi - a and j % 2 == 1)) else j
        assert (orc.round_to_bf16(float(v)) & 0x7FFF) == pick


def _tiny_index_case(seed, T, K, H, R, stride, wdtype, n_invalid, nan_rows=2):
    rng = np.random.Generator(np.random.PCG64(seed))
    store = wl.normal_bf16(rng, (R + nan_rows, stride))
    # spread magnitudes so rounding inside the chain matters
    scale_bits = wl.to_bf16_bits(np.exp2(rng.integers(-6, 7, size=(R + nan_rows, 1))
                                         ).astype(np.float32))
    vals = wl.bf16_bits_to_f32(store) * wl.bf16_bits_to_f32(scale_bits)
    store = wl.to_bf16_bits(vals)
    store[:, H:] = 0x7FC0
    store[R:] = 0x7FC0
    idx = rng.integers(0, R, size=(T, K)).astype(np.int32)
    bad_vals = np.array([-1, np.iinfo(np.int32).min, R, R + 1, 9999, np.iinfo(np.int32).max],
                        dtype=np.int64)
    pos = rng.choice(T * K, size=n_invalid, replace=False)
    idx.reshape(-1)[pos] = rng.choice(bad_vals, size=n_invalid).astype(np.int32)
    w = (rng.standard_normal((T, K)) * np.exp2(rng.integers(-3, 4, size=(T, K)))
         ).astype(np.float32)
    w.reshape(-1)[pos] = np.float32("nan")        # never read
    if wdtype == "bf16":
        w = wl.to_bf16_bits(w)
    return store, R, w, idx


def pin_routed_sum_exact(orc):
    """The FP32 reduction equals, bit for bit, an exact rational model of an
    ascending-slot chain of fused multiply-adds, with invalid slots skipped
    (also with NaN weights, NaN padding columns and NaN rows past num_rows)."""
    cases = [(1, 5, 4, 24, 9, 32, "fp32", 5), (2, 4, 1, 16, 5, 16, "fp32", 1),
             (3, 6, 3, 16, 7, 24, "bf16", 4), (4, 3, 8, 8, 11, 8, "fp32", 6)]
    for seed, T, K, H, R, S, wd, nbad in cases:
        store, R_, w, idx = _tiny_index_case(seed, T, K, H, R, S, wd, nbad)
        got = orc.routed_sum(store, w, idx, H, num_rows=R_)
        want = exact_routed_sum(store, R_, w, idx, H)
        assert f32_equal_pm0(got, want), f"routed sum differs from exact model (case {seed})"


def pin_routed_sum_error_bound(orc):
    """At full width, the FP32 sum is within the FMA-chain error bound of the
    exact sum of w*x over valid slots (exact products in binary64, fsum)."""
    case = wl.tiny(num_tokens=12, num_rows=128, nan_rows_beyond=3)
    acc = orc.routed_sum(case.gemm2_storage, case.expert_weights, case.idx, case.hidden,
                         num_rows=case.num_rows).astype(np.float64)
    g = wl.bf16_bits_to_f32(case.gemm2_storage[:, :case.hidden]).astype(np.float64)
    w = case.expert_weights.astype(np.float64)
    T, K = case.idx.shape
    u = 2.0 ** -24
    for t in range(T):
        terms = [w[t, k] * g[case.idx[t, k]] for k in range(K)
                 if 0 <= case.idx[t, k] < case.num_rows]
        if not terms:
            assert np.all(acc[t] == 0)
            continue
        P = np.stack(terms)
        exact = np.array([math.fsum(P[:, h]) for h in range(case.hidden)])
        bound = 1.01 * len(terms) * u * np.abs(P).sum(axis=0) + 1e-300
        assert np.all(np.abs(acc[t] - exact) <= bound), f"token {t} outside error bound"


def pin_masking_invariants(orc):
    """An invalid slot equals a valid slot with weight 0 and equals the slot
    removed; every out-of-range index value behaves the same; invalid slots'
    NaN weights never reach the output."""
    rng = np.random.Generator(np.random.PCG64(21))
    H, K, T, R = 256, 8, 6, 64
    store = wl.normal_bf16(rng, (R, H))
    idx = rng.permutation(R)[:T * K].reshape(T, K).astype(np.int32)
    w = wl.softmax_rows(rng.standard_normal((T, K)))
    nw = wl.normal_bf16(rng, (H,), std=0.1)
    kw = dict(eps=1e-6, gain_center=1.0, weight_before_norm=False)
    kill = [(0, 3), (1, 0), (2, 7), (4, 1), (4, 2), (5, 0)]
    ref_w = w.copy()
    for t, k in kill:
        ref_w[t, k] = 0.0
    ref_fin = orc.moe_finalize(store, ref_w, idx, H)
    ref_norm = orc.moe_finalize_rmsnorm(store, ref_w, idx, nw, **kw)
    for bad in (-1, np.iinfo(np.int32).min, R, R + 1, 9999, np.iinfo(np.int32).max):
        bidx = idx.copy()
        bw = w.copy()
        for t, k in kill:
            bidx[t, k] = bad
            bw[t, k] = np.float32("nan")
        assert_bits_equal(orc.moe_finalize(store, bw, bidx, H), ref_fin, f"finalize idx={bad}")
        assert_bits_equal(orc.moe_finalize_rmsnorm(store, bw, bidx, nw, **kw), ref_norm,
                          f"rmsnorm idx={bad}")
    # slot removed: move the killed slot to the end and drop it
    t = 3
    bidx = idx.copy()
    bidx[t, 5] = -1
    full = orc.routed_sum(store, w, bidx, H)[t]
    keep = [k for k in range(K) if k != 5]
    part = orc.routed_sum(store, w[t:t + 1, keep], idx[t:t + 1, keep], H)[0]
    assert f32_equal_pm0(full, part)
    # an all-invalid token gives zeros
    zidx = idx.copy()
    zidx[2, :] = -1
    out = orc.moe_finalize(store, w, zidx, H)
    assert np.all((out[2] & 0x7FFF) == 0)


def pin_identity_copy(orc):
    """One valid slot with weight 1 reproduces its row exactly (index map and
    token major); K=1 too."""
    rng = np.random.Generator(np.random.PCG64(22))
    H, R = 512, 40
    store = wl.normal_bf16(rng, (R, H + 64))
    idx = np.full((5, 8), -1, dtype=np.int32)
    rows = rng.choice(R, 5, replace=False)
    w = np.zeros((5, 8), dtype=np.float32)
    for t in range(5):
        k = t % 8
        idx[t, k] = rows[t]
        w[t, k] = 1.0
    out = orc.moe_finalize(store, w, idx, H)
    assert_bits_equal(out, store[rows, :H], "identity copy")
    out1 = orc.moe_finalize(store, np.ones((5, 1), np.float32), rows[:, None].astype(np.int32), H)
    assert_bits_equal(out1, store[rows, :H], "identity copy K=1")
    e = wl.normal_bf16(rng, (6, 1, H))
    outb = orc.beam_moe_finalize(e, np.ones((6, 1), np.float32), 6, routed_scale=1.0)
    assert_bits_equal(outb, e[:, 0, :], "token-major identity copy")


def pin_bf16_weights(orc):
    """BF16 routing weights act exactly as their FP32 widening."""
    case = wl.decode(num_tokens=24, num_rows=256)
    wb = case.expert_weights
    assert wb.dtype == np.uint16
    wf = wl.bf16_bits_to_f32(wb)
    a = orc.routed_sum(case.gemm2, wb, case.idx, case.hidden)
    b = orc.routed_sum(case.gemm2, wf, case.idx, case.hidden)
    assert f32_equal_pm0(a, b)


def pin_finalize_rounds_sum(orc):
    """moe_finalize is the routed FP32 sum rounded by torch's BF16 cast."""
    case = wl.tiny(num_tokens=16)
    acc = orc.routed_sum(case.gemm2, case.expert_weights, case.idx, case.hidden)
    out = orc.moe_finalize(case.gemm2, case.expert_weights, case.idx, case.hidden)
    assert_bits_equal(out, torch_bf16_bits(acc), "moe_finalize")


def _norm_expect(acc, nw_bits, gain_center, eps, wbn):
    """torch rms_norm in float64 on the pinned FP32 sum; g is the FP32 sum of
    the BF16 weight and gain_center."""
    g = (wl.bf16_bits_to_f32(nw_bits) + np.float32(gain_center)).astype(np.float32)
    a = torch.from_numpy(acc.astype(np.float64))
    gt = torch.from_numpy(g.astype(np.float64))
    H = acc.shape[-1]
    if wbn:
        y = torch.nn.functional.rms_norm(a * gt, (H,), eps=eps)
    else:
        y = torch.nn.functional.rms_norm(a, (H,), weight=gt, eps=eps)
    return table_round_to_bf16(y.numpy()).reshape(acc.shape)


def pin_rmsnorm_library(orc):
    """The fused norm equals torch's float64 rms_norm (weight after, or the
    weight folded in before) applied to the FP32 routed sum, within 1 BF16
    ulp and almost always bit-exact."""
    for make, nrows in ((wl.tiny, None), (wl.decode, 512)):
        kw = dict(num_tokens=32, num_rows=256) if nrows is None else dict(num_tokens=48, num_rows=nrows)
        for wbn in (False, True):
            for gc in (1.0, 0.0, -0.25):
                case = make(**kw, weight_before_norm=wbn, gain_center=gc)
                acc = orc.routed_sum(case.gemm2, case.expert_weights, case.idx, case.hidden,
                                     num_rows=case.num_rows)
                want = _norm_expect(acc, case.norm_weight, gc, case.eps, wbn)
                got = orc.moe_finalize_rmsnorm(
                    case.gemm2, case.expert_weights, case.idx, case.norm_weight,
                    eps=case.eps, gain_center=gc, weight_before_norm=wbn,
                    num_rows=case.num_rows)
                assert_within_ulp(got, want, 1, 0.995, f"{case.name} wbn={wbn} gc={gc}")


def pin_rmsnorm_special_case(orc):
    """One valid slot with weight 1 and unit gain is torch's rms_norm of the
    row itself."""
    rng = np.random.Generator(np.random.PCG64(23))
    H, R, T = 4096, 16, 8
    store = wl.normal_bf16(rng, (R, H))
    idx = np.full((T, 8), -1, dtype=np.int32)
    idx[:, 2] = rng.choice(R, T, replace=False)
    w = np.zeros((T, 8), np.float32)
    w[:, 2] = 1.0
    one = np.full(H, 0x3F80, dtype=np.uint16)
    for eps in (1e-6, 1e-2):
        got = orc.moe_finalize_rmsnorm(store, w, idx, one, eps=eps, gain_center=0.0,
                                       weight_before_norm=False)
        rows = torch.from_numpy(wl.bf16_bits_to_f32(store[idx[:, 2]]).astype(np.float64))
        want = table_round_to_bf16(torch.nn.functional.rms_norm(rows, (H,), eps=eps).numpy())
        assert_within_ulp(got, want.reshape(got.shape), 1, 0.999, f"special eps={eps}")


def _const_rows_case(a_rows, weights, H, nw_bits):
    K = len(a_rows)
    store = np.stack([np.full(H, wl.to_bf16_bits(np.array([v], np.float32))[0], np.uint16)
                      for v in a_rows])
    idx = np.arange(K, dtype=np.int32)[None, :]
    w = np.array([weights], dtype=np.float32)
    return store, w, idx, nw_bits


def pin_rmsnorm_closed_forms(orc):
    """Closed forms: a constant sum a gives a/sqrt(a^2+eps)*g; eps sits inside
    the square root; the mean divides by H; gain_center is an FP32 add."""
    H = 256
    one = np.full(H, 0x3F80, np.uint16)
    zero = np.zeros(H, np.uint16)
    # rows 1 and 2 with weights 1/4 and 1/2 sum to 1.25 exactly -> ~1
    store, w, idx, _ = _const_rows_case([1.0, 2.0], [0.25, 0.5], H, one)
    out = orc.moe_finalize_rmsnorm(store, w, idx, zero, eps=1e-6, gain_center=1.0,
                                   weight_before_norm=False)
    assert np.all(out == 0x3F80)
    assert np.all(orc.moe_finalize(store, w, idx, H) == 0x3FA0)      # 1.25
    # eps inside the root: a = 2^-10, eps = 1e-6 -> 0.6987.. -> 0x3F33
    store, w, idx, _ = _const_rows_case([2.0 ** -10], [1.0], H, one)
    out = orc.moe_finalize_rmsnorm(store, w, idx, one, eps=1e-6, gain_center=0.0,
                                   weight_before_norm=False)
    y = 2.0 ** -10 / math.sqrt(2.0 ** -20 + 1e-6)
    assert abs(y - 0.6987) < 1e-3
    assert np.all(out == table_round_to_bf16(np.array([y]))[0])
    # divisor H: half the elements zero -> the others become sqrt(2)
    store = np.zeros((1, H), np.uint16)
    store[0, : H // 2] = 0x3F80
    out = orc.moe_finalize_rmsnorm(store, np.ones((1, 1), np.float32),
                                   np.zeros((1, 1), np.int32), one, eps=1e-6,
                                   gain_center=0.0, weight_before_norm=False)
    want = table_round_to_bf16(np.array([1.0 / math.sqrt(0.5 + 1e-6)]))[0]
    assert np.all(out[0, : H // 2] == want) and want == 0x3FB5
    assert np.all((out[0, H // 2:] & 0x7FFF) == 0)
    # sign follows the sum
    store, w, idx, _ = _const_rows_case([-3.0], [1.0], H, one)
    out = orc.moe_finalize_rmsnorm(store, w, idx, one, eps=1e-6, gain_center=0.0,
                                   weight_before_norm=False)
    assert np.all(out == 0xBF80)
    # gain_center is added in FP32: g = 1 + 2^-12 is not a BF16 value, and
    # with the weight before the norm it reaches the statistics only through
    # the FP32 product; after the norm it multiplies the normalized value.
    H = 4096
    rng = np.random.Generator(np.random.PCG64(24))
    row = wl.normal_bf16(rng, (1, H))
    nw = np.full(H, 0x3F80, np.uint16)
    nw[::2] = 0x4000                                   # 1.0 and 2.0 alternate
    out = orc.moe_finalize_rmsnorm(row, np.ones((1, 1), np.float32),
                                   np.zeros((1, 1), np.int32), nw, eps=1e-6,
                                   gain_center=2.0 ** -12, weight_before_norm=False)
    x = wl.bf16_bits_to_f32(row[0]).astype(np.float64)
    g = wl.bf16_bits_to_f32(nw).astype(np.float64) + 2.0 ** -12
    inv = 1.0 / math.sqrt(float(np.mean(x * x)) + 1e-6)
    assert_within_ulp(out[0], table_round_to_bf16(x * inv * g), 1, 0.99, "gain_center")


def pin_rmsnorm_invariants(orc):
    """With the weight before the norm the output RMS is 1 and scaling the
    weight by 2 changes nothing (eps negligible); with it after, RMS(y) = |c|
    for g = c."""
    case = wl.tiny(num_tokens=16, invalid_frac=0.0)
    nw2 = wl.to_bf16_bits(2 * wl.bf16_bits_to_f32(case.norm_weight))
    outs = []
    for nw in (case.norm_weight, nw2):
        outs.append(orc.moe_finalize_rmsnorm(case.gemm2, case.expert_weights, case.idx, nw,
                                             eps=1e-12, gain_center=0.0,
                                             weight_before_norm=True))
    assert_within_ulp(outs[0], outs[1], 1, 0.999, "scale invariance")
    y = wl.bf16_bits_to_f32(outs[0]).astype(np.float64)
    rms = np.sqrt((y * y).mean(axis=1))
    assert np.all(np.abs(rms - 1) < 5e-3)
    c = 0.75
    cw = np.full(case.hidden, wl.to_bf16_bits(np.array([c], np.float32))[0], np.uint16)
    out = orc.moe_finalize_rmsnorm(case.gemm2, case.expert_weights, case.idx, cw,
                                   eps=1e-6, gain_center=0.0, weight_before_norm=False)
    y = wl.bf16_bits_to_f32(out).astype(np.float64)
    rms = np.sqrt((y * y).mean(axis=1))
    assert np.all(np.abs(rms - c) < 5e-3)


def pin_beam_worked_example(orc):
    """Rounding order: K=1, w = 1 + 7*2^-11, rows of 1.0 and routed_scale 2.5
    give 2.5 (0x4020) when the sum is rounded to BF16 before the scale;
    scaling first would give 2.515625 (0x4021)."""
    H = 256
    e = np.full((3, 1, H), 0x3F80, np.uint16)
    w = np.full((3, 1), 1.0 + 7 * 2.0 ** -11, np.float32)
    out = orc.beam_moe_finalize(e, w, 3, routed_scale=2.5)
    assert np.all(out == 0x4020)
    out = orc.beam_moe_finalize(e, w, 2, routed_scale=1.0)
    assert out.shape == (2, H) and np.all(out == 0x3F80)


def _torch_beam(orc, e_bits, w, live, scale, pw_bits, eps):
    """The beam pipeline with torch CPU ops on the FP32 sum (taken from the
    index-map reduction, pinned above, with an identity map): BF16 cast, FP32
    multiply by the scale, BF16 cast, then float64 rms_norm."""
    C, K, H = e_bits.shape
    idx = np.arange(K, dtype=np.int32)[None, :]
    acc = np.stack([orc.routed_sum(e_bits[t], w[t][None, :].astype(np.float32), idx, H)[0]
                    for t in range(live)])
    r = torch.from_numpy(acc).to(torch.bfloat16)
    s = (r.float() * torch.tensor(scale, dtype=torch.float32)).to(torch.bfloat16)
    s_bits = s.view(torch.int16).numpy().view(np.uint16)
    if eps is None:
        return s_bits
    sw = None if pw_bits is None else torch.from_numpy(
        wl.bf16_bits_to_f32(pw_bits).astype(np.float64))
    y = torch.nn.functional.rms_norm(s.double(), (H,), weight=sw, eps=eps)
    return table_round_to_bf16(y.numpy()).reshape(live, H)


def pin_beam_against_torch_pipeline(orc):
    """Token-major finalize equals torch ops applied in the stated order
    (bit-exact without a norm; within 1 ulp with one); rows and weights past
    live_tokens are NaN and never read."""
    for seed, (C, K, H, live, scale, eps, pws) in enumerate([
            (9, 3, 256, 7, 2.5, None, None), (6, 5, 512, 6, 1.0 / 3.0, None, None),
            (8, 16, 256, 5, 1.0, 1e-6, 0.05), (5, 2, 768, 4, 0.7, 1e-5, None),
            (4, 1, 256, 4, 3.0, 1e-6, 0.05)]):
        case = wl.make_token_major_case(100 + seed, capacity=C, top_k=K, hidden=H,
                                        live_tokens=live, routed_scale=scale,
                                        post_eps=eps, post_weight_std=pws,
                                        poison_dead=True)
        got = orc.beam_moe_finalize(case.expert_outputs, case.expert_weights, live,
                                    routed_scale=scale, post_weight=case.post_weight,
                                    post_eps=eps)
        want = _torch_beam(orc, case.expert_outputs, case.expert_weights, live, scale,
                           case.post_weight, eps)
        if eps is None:
            assert_bits_equal(got, want, f"beam no-norm case {seed}")
        else:
            assert_within_ulp(got, want, 1, 0.99, f"beam norm case {seed}")


def pin_beam_layout(orc):
    """Token-major slot k of token t is the contiguous row [t, k, :]: the no-norm
    beam path at scale 1 equals the index-map finalize with row t*K+k."""
    case = wl.make_token_major_case(7, capacity=12, top_k=4, hidden=512, live_tokens=10)
    C, K, H = case.expert_outputs.shape
    rows = case.expert_outputs.reshape(C * K, H)
    idx = (np.arange(10)[:, None] * K + np.arange(K)[None, :]).astype(np.int32)
    a = orc.beam_moe_finalize(case.expert_outputs, case.expert_weights, 10)
    b = orc.moe_finalize(rows, case.expert_weights[:10], idx, H)
    assert_bits_equal(a, b, "token-major layout")


def pin_standalone_rmsnorm(orc):
    """The standalone norm of BF16 rows equals torch's float64 rms_norm
    (within 1 ulp, almost always exact); on rows whose routed sum is exactly
    the row (one valid slot, weight 1) it equals the fused finalize+norm bit
    for bit; and finalize-then-norm stays within 1 ulp of the fused path."""
    rng = np.random.Generator(np.random.PCG64(41))
    H, T = 2048, 24
    x = wl.normal_bf16(rng, (T, H + 64))
    nw = wl.normal_bf16(rng, (H,), std=0.1)
    for wbn, gc in ((False, 1.0), (True, 0.0), (False, -0.25)):
        got = orc.rmsnorm(x, nw, eps=1e-6, gain_center=gc, weight_before_norm=wbn)
        xa = wl.bf16_bits_to_f32(x[:, :H])
        assert_within_ulp(got, _norm_expect(xa, nw, gc, 1e-6, wbn), 1, 0.995,
                          f"standalone wbn={wbn}")
        idx = np.full((T, 8), -1, np.int32)
        idx[:, 5] = np.arange(T)
        w = np.zeros((T, 8), np.float32)
        w[:, 5] = 1.0
        fused = orc.moe_finalize_rmsnorm(x, w, idx, nw, eps=1e-6, gain_center=gc,
                                         weight_before_norm=wbn)
        assert_bits_equal(got, fused, "norm of exact rows == fused")
    case = wl.tiny(num_tokens=32, num_rows=256)
    fin = orc.moe_finalize(case.gemm2, case.expert_weights, case.idx, case.hidden)
    unf = orc.rmsnorm(fin, case.norm_weight, eps=case.eps, gain_center=case.gain_center,
                      weight_before_norm=case.weight_before_norm)
    fus = orc.moe_finalize_rmsnorm(case.gemm2, case.expert_weights, case.idx, case.norm_weight,
                                   eps=case.eps, gain_center=case.gain_center,
                                   weight_before_norm=case.weight_before_norm)
    assert_within_ulp(unf, fus, 2, 0.5, "unfused vs fused")


def _torch_bf16_add(a_bits, b_bits):
    """torch's BF16 + BF16 (computed in FP32, rounded once to BF16)."""
    a = torch.from_numpy(np.ascontiguousarray(a_bits).view(np.int16)).view(torch.bfloat16)
    b = torch.from_numpy(np.ascontiguousarray(b_bits).view(np.int16)).view(torch.bfloat16)
    return (a + b).view(torch.int16).numpy().view(np.uint16)


def _rmsnorm_expect(bits, weight_bits, eps):
    v = torch.from_numpy(wl.bf16_bits_to_f32(bits).astype(np.float64))
    w = None if weight_bits is None else torch.from_numpy(
        wl.bf16_bits_to_f32(weight_bits).astype(np.float64))
    y = torch.nn.functional.rms_norm(v, (v.shape[-1],), weight=w, eps=eps)
    return table_round_to_bf16(y.numpy()).reshape(bits.shape)


def pin_residual_next_norm(orc):
    """Residual add and next norm (the reading of the off-page consumer):
    zero residual is the identity, the add is torch's BF16 add, the next norm
    is torch's float64 rms_norm of hidden as stored in BF16, the post-norm is
    the beam post-norm, scales[0] multiplies x and scales[1] the residual,
    and the fused op is beam_moe_finalize followed by the consumer."""
    rng = np.random.Generator(np.random.PCG64(51))
    T, H = 12, 1024
    x = wl.normal_bf16(rng, (T, H + 64))
    x[:, H:] = 0x7FC0
    res = wl.normal_bf16(rng, (T, H))
    pw = wl.normal_bf16(rng, (H,), mean=1.0, std=0.05)
    nw = wl.normal_bf16(rng, (H,), mean=1.0, std=0.1)
    zero = np.zeros((T, H), np.uint16)
    hid, nrm = orc.beam_norm_residual_norm(x, zero)
    assert nrm is None
    assert_bits_equal(hid, x[:, :H], "zero residual")
    hid, nrm = orc.beam_norm_residual_norm(x, res, next_weight=nw, next_eps=1e-6)
    assert_within_ulp(hid, _torch_bf16_add(x[:, :H], res), 1, 0.999, "residual add")
    assert_within_ulp(nrm, _rmsnorm_expect(hid, nw, 1e-6), 1, 0.99, "next norm")
    hid, nrm = orc.beam_norm_residual_norm(x, res, next_eps=1e-5)
    assert_within_ulp(nrm, _rmsnorm_expect(hid, None, 1e-5), 1, 0.99, "next norm, no weight")
    hid, _ = orc.beam_norm_residual_norm(x, zero, post_weight=pw, post_eps=1e-6)
    post = _rmsnorm_expect(x[:, :H], pw, 1e-6)
    assert_within_ulp(hid, post, 1, 0.99, "post norm")
    # the post-normed value is rounded to BF16 before the residual add
    hid, _ = orc.beam_norm_residual_norm(x, res, post_weight=pw, post_eps=1e-6)
    assert_within_ulp(hid, _torch_bf16_add(post, res), 1, 0.99, "post norm, then add")
    hid, _ = orc.beam_norm_residual_norm(x, res, scales=(2.0, 0.0))
    assert_bits_equal(hid, table_round_to_bf16(2.0 * wl.bf16_bits_to_f32(x[:, :H])).reshape(T, H),
                      "scales[0] scales x")
    hid, _ = orc.beam_norm_residual_norm(x, res, scales=(0.0, 1.0))
    assert_bits_equal(hid, res, "scales[1] scales the residual")
    # fused == finalize then consumer
    case = wl.make_token_major_case(52, capacity=14, top_k=4, hidden=H, live_tokens=T,
                                    routed_scale=1.5, post_eps=1e-6, post_weight_std=0.05,
                                    poison_dead=True)
    fin = orc.beam_moe_finalize(case.expert_outputs, case.expert_weights, T, 1.5,
                                case.post_weight, 1e-6)
    want_h, want_n = orc.beam_norm_residual_norm(fin, res, next_weight=nw, next_eps=1e-6,
                                                 scales=(0.5, 2.0))
    got_h, got_n = orc.beam_moe_finalize_norm_residual_norm(
        case.expert_outputs, case.expert_weights, res, case.post_weight, 1e-6, nw, 1e-6,
        (0.5, 2.0), 1.5)
    assert_bits_equal(got_h, want_h, "fused hidden")
    assert_bits_equal(got_n, want_n, "fused normalized")


ALL_PINS = [pin_bf16_widening, pin_rne_against_torch, pin_rne_binary64_single_rounding,
            pin_routed_sum_exact, pin_routed_sum_error_bound, pin_masking_invariants,
            pin_identity_copy, pin_bf16_weights, pin_finalize_rounds_sum,
            pin_rmsnorm_library, pin_rmsnorm_special_case, pin_rmsnorm_closed_forms,
            pin_rmsnorm_invariants, pin_beam_worked_example,
            pin_beam_against_torch_pipeline, pin_beam_layout, pin_standalone_rmsnorm,
            pin_residual_next_norm]
