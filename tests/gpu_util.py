"""Helpers shared by the GPU tests: numpy <-> device tensors and running the
library's entry points on the seeded cases of workloads.py."""
from __future__ import annotations

import numpy as np
import torch

import workloads as wl


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
