"""Helpers shared by the GPU tests: numpy <-> device tensors, and running the
library's entry points and the oracle side by side on the seeded cases of
workloads.py."""
from __future__ import annotations

import numpy as np
import torch

import moe_expert_output_finalize_amd as mf
import oracle
import workloads as wl
from oracle_pins import assert_bits_equal, assert_within_ulp

NORM_MIN_EXACT = 0.98      # sanity floor on the bit-exact share of normalised outputs


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def dev_weights(w: np.ndarray, device="cuda") -> torch.Tensor:
    if w.dtype == np.uint16:
        return dev_bf16(w, device)
    return torch.from_numpy(np.ascontiguousarray(w)).to(device)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


class IndexMapOnDevice:
    """Device copies of an IndexMapCase; `gemm2` is the [num_rows, stride] view of
    the storage (extra NaN rows past num_rows stay allocated behind it)."""

    def __init__(self, case: wl.IndexMapCase, device="cuda"):
        self.case = case
        self.storage = dev_bf16(case.gemm2_storage, device)
        self.gemm2 = self.storage[: case.num_rows]
        self.weights = dev_weights(case.expert_weights, device)
        self.idx = torch.from_numpy(case.idx).to(device)
        self.norm_weight = dev_bf16(case.norm_weight, device)

    def new_output(self, fill_bits: int = 0x7FC0) -> torch.Tensor:
        out = torch.empty((self.case.num_tokens, self.case.hidden), dtype=torch.int16,
                          device=self.storage.device)
        out.fill_(np.int16(np.uint16(fill_bits).view(np.int16)))
        return out.view(torch.bfloat16)


class TokenMajorOnDevice:
    def __init__(self, case: wl.TokenMajorCase, device="cuda"):
        self.case = case
        self.expert_outputs = dev_bf16(case.expert_outputs, device)
        self.weights = torch.from_numpy(case.expert_weights).to(device)
        self.post_weight = None if case.post_weight is None else dev_bf16(case.post_weight, device)

    def new_output(self, live: int | None = None) -> torch.Tensor:
        live = self.case.live_tokens if live is None else live
        out = torch.full((live, self.case.hidden), float("nan"), dtype=torch.bfloat16,
                         device=self.expert_outputs.device)
        return out


# --------------------------------------------------------------- runners ----

def sync():
    torch.cuda.synchronize()


def gpu_rmsnorm(d: IndexMapOnDevice, **kw) -> np.ndarray:
    c = d.case
    args = dict(eps=c.eps, gain_center=c.gain_center, weight_before_norm=c.weight_before_norm)
    args.update(kw)
    out = d.new_output()
    mf.moe_finalize_rmsnorm(d.gemm2, d.weights, d.idx, d.norm_weight, out, **args)
    sync()
    return host_bits(out)


def oracle_rmsnorm(c: wl.IndexMapCase, **kw) -> np.ndarray:
    args = dict(eps=c.eps, gain_center=c.gain_center, weight_before_norm=c.weight_before_norm)
    args.update(kw)
    return oracle.moe_finalize_rmsnorm(c.gemm2, c.expert_weights, c.idx, c.norm_weight, **args)


def gpu_finalize(d: IndexMapOnDevice) -> np.ndarray:
    out = d.new_output()
    mf.moe_finalize(d.gemm2, d.weights, d.idx, out)
    sync()
    return host_bits(out)


def oracle_finalize(c: wl.IndexMapCase) -> np.ndarray:
    return oracle.moe_finalize(c.gemm2, c.expert_weights, c.idx, c.hidden)


def gpu_beam(d: TokenMajorOnDevice, live=None) -> np.ndarray:
    c = d.case
    out = d.new_output(live)
    mf.beam_moe_finalize(d.expert_outputs, d.weights, out, c.routed_scale, d.post_weight,
                         c.post_eps)
    sync()
    return host_bits(out)


def oracle_beam(c: wl.TokenMajorCase, live=None) -> np.ndarray:
    live = c.live_tokens if live is None else live
    return oracle.beam_moe_finalize(c.expert_outputs, c.expert_weights, live, c.routed_scale,
                                    c.post_weight, c.post_eps)


# ------------------------------- finalize -> residual -> next norm ----

def residual_case(seed, capacity, top_k, hidden, tokens, post, post_w, nxt, next_w, scales,
                  routed_scale=1.0):
    c = wl.make_token_major_case(seed, capacity=capacity, top_k=top_k, hidden=hidden,
                                 live_tokens=tokens, routed_scale=routed_scale,
                                 post_eps=1e-6 if post else None,
                                 post_weight_std=0.05 if (post and post_w) else None,
                                 poison_dead=True)
    rng = np.random.Generator(np.random.PCG64(seed + 7))
    res = wl.normal_bf16(rng, (tokens, hidden))
    nw = wl.normal_bf16(rng, (hidden,), mean=1.0, std=0.1) if (nxt and next_w) else None
    return c, res, nw, (1e-6 if nxt else None), scales


def check_residual(c, res, nw, next_eps, scales, what):
    """Fused op on the GPU vs the oracle.  With a post-norm the finalized
    value y is only within 1 ulp of the oracle's, and the residual add can
    amplify that by cancellation, so the comparison is split: the GPU's y
    against the oracle's finalize, the GPU's hidden / normalized against the
    oracle's consumer applied to the GPU's own y, and the fused kernel against
    the two-step GPU path bit for bit.  Without a post-norm y is exact and the
    fused result is also compared with the oracle's fused op directly."""
    d = TokenMajorOnDevice(c)
    T = res.shape[0]
    resd = dev_bf16(res)
    nwd = None if nw is None else dev_bf16(nw)
    h, n = mf.beam_moe_finalize_norm_residual_norm(d.expert_outputs, d.weights, resd,
                                                   d.post_weight, c.post_eps, nwd, next_eps,
                                                   scales, c.routed_scale)
    fin = d.new_output(T)
    mf.beam_moe_finalize(d.expert_outputs, d.weights, fin, c.routed_scale, d.post_weight,
                         c.post_eps)
    h2, n2 = mf.beam_norm_residual_norm(fin, resd, None, None, nwd, next_eps, scales)
    sync()
    y = host_bits(fin)
    want_y = oracle_beam(c, T)
    if c.post_eps is None:
        assert_bits_equal(y, want_y, f"{what} y")
    else:
        assert_within_ulp(y, want_y, 1, NORM_MIN_EXACT, f"{what} y")
    got_h, got_n = host_bits(h), (None if n is None else host_bits(n))
    assert (got_n is None) == (next_eps is None)
    ch, cn = oracle.beam_norm_residual_norm(y, res, None, None, nw, next_eps, scales)
    # hidden is one rounding of scale_x * y + scale_res * residual on both
    # sides, from the same y: bit for bit
    assert_bits_equal(got_h, ch, f"{what} hidden")
    if cn is not None:
        assert_within_ulp(got_n, cn, 1, NORM_MIN_EXACT, f"{what} normalized")
    if c.post_eps is None:
        fh, fn = oracle.beam_moe_finalize_norm_residual_norm(
            c.expert_outputs, c.expert_weights, res, c.post_weight, c.post_eps, nw, next_eps,
            scales, c.routed_scale)
        assert_bits_equal(got_h, fh, f"{what} hidden vs fused oracle")
        if fn is not None:
            assert_within_ulp(got_n, fn, 1, NORM_MIN_EXACT, f"{what} normalized vs fused oracle")
    assert_bits_equal(got_h, host_bits(h2), f"{what} fused vs unfused hidden")
    if got_n is not None:
        assert_bits_equal(got_n, host_bits(n2), f"{what} fused vs unfused normalized")
