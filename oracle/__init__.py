"""CPU oracle for the MoE expert-output finalize path (numpy front end).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this package; the product library never does.
It shares no code with the GPU library: the arithmetic lives in ``oracle.c``
(plain C, compiled with gcc without fast-math or contraction) and this module
only marshals numpy arrays into it.

What each function computes, and the readings of points the pages leave open,
are stated in ``oracle.c``; the sources are the FlashInfer page
"flashinfer.comm.tp_moe_finalize_rmsnorm" (description and Parameters) and the
vLLM page "vllm.models.beam.nvidia.moe_finalize" (beam_moe_finalize).

BF16 tensors are passed as numpy ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc; returns the path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
        lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f32.restype = f32
        lib.oracle_round_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_to_bf16.restype = ctypes.c_uint16
        lib.oracle_routed_sum.argtypes = [vp, i64, i64, vp, i32, vp, vp, i64, i32, i32]
        lib.oracle_moe_finalize.argtypes = [vp, i64, i64, vp, i32, vp, vp, i64, i32, i32]
        lib.oracle_moe_finalize_rmsnorm.argtypes = [vp, i64, i64, vp, i32, vp, vp, vp,
                                                    i64, i32, i32, f32, f32, i32]
        lib.oracle_beam_moe_finalize.argtypes = [vp, i64, i32, i32, vp, vp, i64, vp,
                                                 f32, f32, i32]
        lib.oracle_rmsnorm.argtypes = [vp, i64, vp, vp, i64, i32, f32, f32, i32]
        lib.oracle_beam_norm_residual_norm.argtypes = [vp, i64, vp, vp, vp, vp, vp, i64, i32,
                                                       f32, f32, f32, f32, i32, i32]
        lib.oracle_beam_moe_finalize_norm_residual_norm.argtypes = [
            vp, i64, i32, i32, vp, vp, vp, vp, vp, vp, i64, f32, f32, f32, f32, f32, i32, i32]
        for name in ("oracle_routed_sum", "oracle_moe_finalize", "oracle_rmsnorm",
                     "oracle_moe_finalize_rmsnorm", "oracle_beam_moe_finalize",
                     "oracle_beam_norm_residual_norm",
                     "oracle_beam_moe_finalize_norm_residual_norm"):
            getattr(lib, name).restype = i32
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None) -> int | None:
    return None if a is None else a.ctypes.data


def _check(rc: int, name: str) -> None:
    if rc != 0:
        raise ValueError(f"{name}: oracle rejected its arguments (rc={rc})")


def _rows_view(gemm2_permuted: np.ndarray, hidden: int):
    """(array, num_rows, row_stride) of a 2-D uint16 row matrix whose last
    dimension has unit stride; rows may be padded beyond ``hidden``."""
    g = gemm2_permuted
    assert g.dtype == np.uint16 and g.ndim == 2 and g.strides[1] == 2
    assert g.shape[1] >= hidden
    return g, g.shape[0], g.strides[0] // 2


def _weights(weights: np.ndarray):
    w = np.ascontiguousarray(weights)
    if w.dtype == np.float32:
        return w, 1
    if w.dtype == np.uint16:          # BF16 bit patterns
        return w, 0
    raise TypeError("expert_weights must be float32 or uint16 (BF16 bits)")


# ------------------------------------------------------------------ scalars --

def bf16_to_f32(bits: int) -> float:
    return float(_load().oracle_bf16_to_f32(int(bits)))


def round_to_bf16(x: float) -> int:
    """Nearest BF16 bit pattern of a binary64 value (ties to even)."""
    return int(_load().oracle_round_to_bf16(float(x)))


# ------------------------------------------------------------- index map -----

def routed_sum(gemm2_permuted, expert_weights, expanded_idx_to_permuted_idx,
               hidden: int, num_rows: int | None = None) -> np.ndarray:
    """FP32 routed sums [T, hidden] (float32) of the index-map layout."""
    g, rows, stride = _rows_view(gemm2_permuted, hidden)
    rows = rows if num_rows is None else num_rows
    w, is32 = _weights(expert_weights)
    idx = np.ascontiguousarray(expanded_idx_to_permuted_idx, dtype=np.int32)
    T, K = idx.shape
    assert w.shape == (T, K)
    out = np.empty((T, hidden), dtype=np.float32)
    _check(_load().oracle_routed_sum(_ptr(g), rows, stride, _ptr(w), is32, _ptr(idx),
                                     _ptr(out), T, hidden, K), "routed_sum")
    return out


def moe_finalize(gemm2_permuted, expert_weights, expanded_idx_to_permuted_idx,
                 hidden: int, num_rows: int | None = None) -> np.ndarray:
    """BF16 bits [T, hidden] of bf16(routed FP32 sum)."""
    g, rows, stride = _rows_view(gemm2_permuted, hidden)
    rows = rows if num_rows is None else num_rows
    w, is32 = _weights(expert_weights)
    idx = np.ascontiguousarray(expanded_idx_to_permuted_idx, dtype=np.int32)
    T, K = idx.shape
    assert w.shape == (T, K)
    out = np.empty((T, hidden), dtype=np.uint16)
    _check(_load().oracle_moe_finalize(_ptr(g), rows, stride, _ptr(w), is32, _ptr(idx),
                                       _ptr(out), T, hidden, K), "moe_finalize")
    return out


def moe_finalize_rmsnorm(gemm2_permuted, expert_weights, expanded_idx_to_permuted_idx,
                         norm_weight, *, eps: float, gain_center: float,
                         weight_before_norm: bool, num_rows: int | None = None) -> np.ndarray:
    """BF16 bits [T, hidden] of the finalize fused with per-token RMSNorm."""
    nw = np.ascontiguousarray(norm_weight, dtype=np.uint16)
    hidden = nw.shape[0]
    g, rows, stride = _rows_view(gemm2_permuted, hidden)
    rows = rows if num_rows is None else num_rows
    w, is32 = _weights(expert_weights)
    idx = np.ascontiguousarray(expanded_idx_to_permuted_idx, dtype=np.int32)
    T, K = idx.shape
    assert w.shape == (T, K)
    out = np.empty((T, hidden), dtype=np.uint16)
    _check(_load().oracle_moe_finalize_rmsnorm(
        _ptr(g), rows, stride, _ptr(w), is32, _ptr(idx), _ptr(nw), _ptr(out), T,
        hidden, K, float(eps), float(gain_center), int(bool(weight_before_norm))),
        "moe_finalize_rmsnorm")
    return out


def rmsnorm(x, norm_weight, *, eps: float, gain_center: float,
            weight_before_norm: bool) -> np.ndarray:
    """BF16 bits [T, hidden] of the standalone RMSNorm of BF16 rows ``x``
    (uint16 [T, >= hidden], unit stride in the last dimension)."""
    nw = np.ascontiguousarray(norm_weight, dtype=np.uint16)
    hidden = nw.shape[0]
    g, T, stride = _rows_view(x, hidden)
    out = np.empty((T, hidden), dtype=np.uint16)
    _check(_load().oracle_rmsnorm(_ptr(g), stride, _ptr(nw), _ptr(out), T, hidden, float(eps),
                                  float(gain_center), int(bool(weight_before_norm))),
           "rmsnorm")
    return out


# ----------------------------------------------------------- token major -----

def beam_moe_finalize(expert_outputs, expert_weights, live_tokens: int,
                      routed_scale: float = 1.0, post_weight=None,
                      post_eps: float | None = None) -> np.ndarray:
    """BF16 bits [live_tokens, hidden] of the token-major finalize."""
    e = expert_outputs
    assert e.dtype == np.uint16 and e.ndim == 3 and e.flags.c_contiguous
    capacity, K, H = e.shape
    w = np.ascontiguousarray(expert_weights, dtype=np.float32)
    assert w.ndim == 2 and w.shape[1] == K and w.shape[0] >= live_tokens
    pw = None if post_weight is None else np.ascontiguousarray(post_weight, dtype=np.uint16)
    if pw is not None:
        assert post_eps is not None and pw.shape == (H,)
    out = np.empty((live_tokens, H), dtype=np.uint16)
    _check(_load().oracle_beam_moe_finalize(
        _ptr(e), capacity, K, H, _ptr(w), _ptr(out), int(live_tokens), _ptr(pw),
        float(routed_scale), float(post_eps or 0.0), int(post_eps is not None)),
        "beam_moe_finalize")
    return out


# --------------------------------------- residual add + next norm (f1) -------
# The consumer these two follow is not defined on the pages; see oracle.c for
# the reading (PARITY UNPINNED against the pages).

def beam_norm_residual_norm(x, residual, post_weight=None, post_eps=None, next_weight=None,
                            next_eps=None, scales=None):
    """(hidden, normalized or None) BF16 bits of post-norm -> residual add ->
    next norm on BF16 rows ``x`` (uint16 [T, >= H]) and ``residual`` ([T, H])."""
    r = np.ascontiguousarray(residual, dtype=np.uint16)
    T, H = r.shape
    g, T2, stride = _rows_view(x, H)
    assert T2 == T
    pw = None if post_weight is None else np.ascontiguousarray(post_weight, dtype=np.uint16)
    nw = None if next_weight is None else np.ascontiguousarray(next_weight, dtype=np.uint16)
    hid = np.empty((T, H), dtype=np.uint16)
    nrm = np.empty((T, H), dtype=np.uint16) if next_eps is not None else None
    sx, sr = scales if scales is not None else (1.0, 1.0)
    _check(_load().oracle_beam_norm_residual_norm(
        _ptr(g), stride, _ptr(r), _ptr(pw), _ptr(nw), _ptr(hid), _ptr(nrm), T, H,
        float(post_eps or 0.0), float(next_eps or 0.0), float(sx), float(sr),
        int(post_eps is not None), int(next_eps is not None)), "beam_norm_residual_norm")
    return hid, nrm


def beam_moe_finalize_norm_residual_norm(expert_outputs, expert_weights, residual,
                                         post_weight=None, post_eps=None, next_weight=None,
                                         next_eps=None, scales=None, routed_scale=1.0):
    """(hidden, normalized or None) BF16 bits of the token-major finalize
    followed by the residual add and next norm, for residual.shape[0] tokens."""
    e = expert_outputs
    assert e.dtype == np.uint16 and e.ndim == 3 and e.flags.c_contiguous
    capacity, K, H = e.shape
    r = np.ascontiguousarray(residual, dtype=np.uint16)
    T = r.shape[0]
    w = np.ascontiguousarray(expert_weights, dtype=np.float32)
    assert w.shape[1] == K and w.shape[0] >= T and r.shape == (T, H)
    pw = None if post_weight is None else np.ascontiguousarray(post_weight, dtype=np.uint16)
    nw = None if next_weight is None else np.ascontiguousarray(next_weight, dtype=np.uint16)
    hid = np.empty((T, H), dtype=np.uint16)
    nrm = np.empty((T, H), dtype=np.uint16) if next_eps is not None else None
    sx, sr = scales if scales is not None else (1.0, 1.0)
    _check(_load().oracle_beam_moe_finalize_norm_residual_norm(
        _ptr(e), capacity, K, H, _ptr(w), _ptr(r), _ptr(pw), _ptr(nw), _ptr(hid), _ptr(nrm), T,
        float(routed_scale), float(post_eps or 0.0), float(next_eps or 0.0), float(sx),
        float(sr), int(post_eps is not None), int(next_eps is not None)),
        "beam_moe_finalize_norm_residual_norm")
    return hid, nrm
