"""Seeded synthetic inputs for the MoE finalize path.

This module only draws random numbers and arranges them into the layouts the
finalize entry points take.  It holds none of the method's arithmetic, so both
the CPU oracle and the GPU library can be fed from it.  BF16 tensors are numpy
``uint16`` bit patterns; float32 -> BF16 conversion of the drawn values is
torch's CPU cast (round to nearest even).

The five named workloads mirror the shapes, dtypes and value distributions
the finalize pages' parameter contracts imply:

  tiny     index map, T=16,   H=4096, K=8, 128 rows, FP32 weights, 5 % invalid
  decode   index map, T=256,  H=4096, K=8, 2048 rows with row stride 4160,
           BF16 weights, 2 % invalid, weight applied before the norm
  prefill  index map, T=8192, H=4096, K=8, 65536 rows grouped by expert
           (256 experts, Zipf(1.1) popularity), FP32 weights
  beam4    token major, capacity 4096, K=8,  H=7168, 3000 live, scale 2.5,
           no norm
  beam5    token major, capacity 16384, K=16, H=2048, 16000 live, post norm

and, for the index-map path over the token-major path's envelope, the two
beam shapes through an expert-grouped index map (imap7168, imap2048k16).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

_CHUNK = 1 << 24


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> BF16 bit patterns (uint16) via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, mean: float = 0.0,
                std: float = 1.0) -> np.ndarray:
    """BF16 bits of N(mean, std^2) draws, generated in fixed-size chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        x = rng.standard_normal(m, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        if mean != 0.0:
            x += np.float32(mean)
        out[s:s + m] = to_bf16_bits(x)
    return out.reshape(shape)


def softmax_rows(logits: np.ndarray) -> np.ndarray:
    """Row-wise softmax in float64, returned as float32 (routing weights)."""
    z = logits.astype(np.float64)
    z -= z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


@dataclass
class IndexMapCase:
    """Inputs of moe_finalize / moe_finalize_rmsnorm (index-map layout)."""
    gemm2_storage: np.ndarray          # uint16 [alloc_rows, row_stride]
    num_rows: int                      # rows an index may select
    hidden: int
    expert_weights: np.ndarray         # float32 or uint16(BF16) [T, K]
    idx: np.ndarray                    # int32 [T, K]
    norm_weight: np.ndarray            # uint16 [hidden]
    eps: float
    gain_center: float
    weight_before_norm: bool
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def num_tokens(self) -> int:
        return self.idx.shape[0]

    @property
    def top_k(self) -> int:
        return self.idx.shape[1]

    @property
    def row_stride(self) -> int:
        return self.gemm2_storage.shape[1]

    @property
    def gemm2(self) -> np.ndarray:
        """The [num_rows, row_stride] view an index may select from."""
        return self.gemm2_storage[: self.num_rows]

    @property
    def weights_dtype(self) -> str:
        return "fp32" if self.expert_weights.dtype == np.float32 else "bf16"


@dataclass
class TokenMajorCase:
    """Inputs of beam_moe_finalize (token-major layout)."""
    expert_outputs: np.ndarray         # uint16 [capacity, K, H]
    expert_weights: np.ndarray         # float32 [>= live, K]
    live_tokens: int
    routed_scale: float
    post_weight: np.ndarray | None     # uint16 [H] or None
    post_eps: float | None
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def capacity(self) -> int:
        return self.expert_outputs.shape[0]

    @property
    def top_k(self) -> int:
        return self.expert_outputs.shape[1]

    @property
    def hidden(self) -> int:
        return self.expert_outputs.shape[2]


def zipf_grouped_index_map(rng: np.random.Generator, num_tokens: int, top_k: int,
                           num_experts: int, zipf_s: float) -> np.ndarray:
    """Index map whose physical rows are grouped by expert.

    Expert e has popularity proportional to (e+1)^-zipf_s; each token draws
    top_k distinct experts by weighted sampling without replacement (Gumbel
    top-k over log-popularity).  All (token, slot) pairs are then ordered by
    (expert, token); a pair's rank is its physical row, so the map is a
    permutation of 0..T*K-1 in which a popular expert's tokens are adjacent.
    """
    logp = -zipf_s * np.log(np.arange(1, num_experts + 1, dtype=np.float64))
    scores = logp[None, :] + rng.gumbel(size=(num_tokens, num_experts))
    experts = np.argsort(-scores, axis=1, kind="stable")[:, :top_k]
    tok = np.repeat(np.arange(num_tokens), top_k)
    exp_flat = experts.reshape(-1)
    order = np.lexsort((tok, exp_flat))             # by expert, then token
    idx = np.empty(num_tokens * top_k, dtype=np.int64)
    idx[order] = np.arange(num_tokens * top_k)
    return idx.reshape(num_tokens, top_k).astype(np.int32)


def make_index_map_case(seed: int, *, num_tokens: int, hidden: int = 4096,
                        top_k: int = 8, num_rows: int | None = None,
                        row_stride: int | None = None, weights_dtype: str = "fp32",
                        logit_std: float = 1.0, invalid_frac: float = 0.0,
                        grouping: str = "permutation", num_experts: int = 256,
                        zipf_s: float = 1.1, norm_weight_mean: float = 0.0,
                        norm_weight_std: float = 0.1, eps: float = 1e-6,
                        gain_center: float = 1.0, weight_before_norm: bool = False,
                        poison: bool = False, nan_rows_beyond: int = 0,
                        name: str = "") -> IndexMapCase:
    """Seeded index-map case.

    poison          fill padding columns [hidden, row_stride) with NaN
    nan_rows_beyond allocate that many extra NaN rows after num_rows; invalid
                    indices then point into them (num_rows, num_rows+1, ...)
    """
    rng = _rng(seed)
    T, K, H = num_tokens, top_k, hidden
    R = T * K if num_rows is None else num_rows
    S = H if row_stride is None else row_stride
    assert S >= H and S % 8 == 0
    alloc = R + nan_rows_beyond
    g = normal_bf16(rng, (alloc, S))
    nan_bits = np.uint16(0x7FC0)
    if poison and S > H:
        g[:, H:] = nan_bits
    if nan_rows_beyond:
        g[R:] = nan_bits

    if grouping == "permutation":
        assert R >= T * K
        idx = rng.permutation(R)[: T * K].reshape(T, K).astype(np.int32)
    elif grouping == "zipf":
        assert R == T * K
        idx = zipf_grouped_index_map(rng, T, K, num_experts, zipf_s)
    else:
        raise ValueError(grouping)

    n_bad = int(round(invalid_frac * T * K))
    if n_bad:
        pos = rng.choice(T * K, size=n_bad, replace=False)
        far = 9999 if 9999 >= R else R
        if nan_rows_beyond:
            far = R + 1 if nan_rows_beyond > 1 else R
        coin = rng.integers(0, 2, size=n_bad)
        flat = idx.reshape(-1)
        flat[pos] = np.where(coin == 0, -1, far).astype(np.int32)

    w = softmax_rows(rng.standard_normal((T, K)) * logit_std)
    if weights_dtype == "bf16":
        w = to_bf16_bits(w)
    else:
        assert weights_dtype == "fp32"
    nw = normal_bf16(rng, (H,), mean=norm_weight_mean, std=norm_weight_std)
    return IndexMapCase(g, R, H, w, idx, nw, eps, gain_center, weight_before_norm,
                        name=name, meta=dict(seed=seed, grouping=grouping,
                                             invalid=n_bad))


def make_token_major_case(seed: int, *, capacity: int, top_k: int, hidden: int,
                          live_tokens: int, weights: str = "softmax",
                          routed_scale: float = 1.0, post_eps: float | None = None,
                          post_weight_std: float | None = None,
                          poison_dead: bool = False, name: str = "") -> TokenMajorCase:
    """Seeded token-major case.

    weights      "softmax" (of N(0,1) logits) or "uniform" (U(0,1) / row sum)
    poison_dead  set rows and weights of tokens >= live_tokens to NaN
    """
    rng = _rng(seed)
    C, K, H = capacity, top_k, hidden
    e = normal_bf16(rng, (C, K, H))
    if weights == "softmax":
        w = softmax_rows(rng.standard_normal((C, K)))
    elif weights == "uniform":
        u = rng.random((C, K))
        w = (u / u.sum(axis=1, keepdims=True)).astype(np.float32)
    else:
        raise ValueError(weights)
    pw = None
    if post_weight_std is not None:
        pw = normal_bf16(rng, (H,), mean=1.0, std=post_weight_std)
    if poison_dead and live_tokens < C:
        e[live_tokens:] = np.uint16(0x7FC0)
        w[live_tokens:] = np.float32("nan")
    return TokenMajorCase(e, w, live_tokens, routed_scale, pw, post_eps, name=name,
                          meta=dict(seed=seed))


# ----------------------------------------------------------- named configs ---

def tiny(**kw) -> IndexMapCase:
    args = dict(num_tokens=16, num_rows=128, weights_dtype="fp32", logit_std=1.0,
                invalid_frac=6 / 128, eps=1e-6, gain_center=1.0,
                weight_before_norm=False, norm_weight_mean=0.0, norm_weight_std=0.1,
                name="tiny")
    args.update(kw)
    return make_index_map_case(0, **args)


def decode(**kw) -> IndexMapCase:
    args = dict(num_tokens=256, num_rows=2048, row_stride=4160, weights_dtype="bf16",
                logit_std=1.0, invalid_frac=41 / 2048, eps=1e-5, gain_center=0.0,
                weight_before_norm=True, norm_weight_mean=1.0, norm_weight_std=0.1,
                name="decode")
    args.update(kw)
    return make_index_map_case(1, **args)


def prefill(**kw) -> IndexMapCase:
    args = dict(num_tokens=8192, weights_dtype="fp32", logit_std=2.0,
                grouping="zipf", num_experts=256, zipf_s=1.1, eps=1e-6,
                gain_center=1.0, weight_before_norm=False, norm_weight_mean=0.0,
                norm_weight_std=0.1, name="prefill")
    args.update(kw)
    return make_index_map_case(2, **args)


def beam4(**kw) -> TokenMajorCase:
    args = dict(capacity=4096, top_k=8, hidden=7168, live_tokens=3000,
                weights="uniform", routed_scale=2.5, post_eps=None, name="beam4")
    args.update(kw)
    return make_token_major_case(3, **args)


def beam5(**kw) -> TokenMajorCase:
    args = dict(capacity=16384, top_k=16, hidden=2048, live_tokens=16000,
                weights="softmax", routed_scale=1.0, post_eps=1e-6,
                post_weight_std=0.05, name="beam5")
    args.update(kw)
    return make_token_major_case(4, **args)


def imap7168(**kw) -> IndexMapCase:
    """Index-map finalize+RMSNorm at the beam4 shape: 3000 tokens, hidden
    7168, top-k 8, rows grouped by expert (Zipf 1.1 over 256 experts)."""
    args = dict(num_tokens=3000, hidden=7168, top_k=8, weights_dtype="fp32", logit_std=2.0,
                grouping="zipf", num_experts=256, zipf_s=1.1, eps=1e-6, gain_center=1.0,
                weight_before_norm=False, norm_weight_mean=0.0, norm_weight_std=0.1,
                name="imap7168")
    args.update(kw)
    return make_index_map_case(5, **args)


def imap2048k16(**kw) -> IndexMapCase:
    """Index-map finalize+RMSNorm at the beam5 shape: 16000 tokens, hidden
    2048, top-k 16, rows grouped by expert (Zipf 1.1 over 256 experts)."""
    args = dict(num_tokens=16000, hidden=2048, top_k=16, weights_dtype="fp32",
                logit_std=1.0, grouping="zipf", num_experts=256, zipf_s=1.1, eps=1e-6,
                gain_center=0.0, weight_before_norm=True, norm_weight_mean=1.0,
                norm_weight_std=0.1, name="imap2048k16")
    args.update(kw)
    return make_index_map_case(6, **args)


CONFIGS = {"tiny": tiny, "decode": decode, "prefill": prefill,
           "beam4": beam4, "beam5": beam5, "imap7168": imap7168,
           "imap2048k16": imap2048k16}
