"""MoE expert-output finalize for MI355X (gfx950): Python binding.

Thin ctypes layer over ``libmoe_finalize.so`` (C ABI in
``include/moe_finalize.h``).  It only marshals torch tensors into pointers,
sizes and the current HIP stream; every step of the computation runs in the
library's HIP kernels.  There is no fallback: if the library is not built,
importing this package raises.

Entry points (same names as the C ABI):
  moe_finalize_rmsnorm  index-map finalize + per-token RMSNorm
                        (FlashInfer "flashinfer.comm.tp_moe_finalize_rmsnorm")
  moe_finalize          index-map finalize without a norm
  beam_moe_finalize     token-major finalize with BF16 rounding points and an
                        optional RMSNorm (vLLM "vllm.models.beam.nvidia.moe_finalize")
  mf_rmsnorm            standalone RMSNorm of BF16 rows (the second step of the
                        unfused baseline moe_finalize -> mf_rmsnorm)
  beam_moe_finalize_norm_residual_norm
                        token-major finalize fused with the residual add and the
                        next norm (vLLM page, same function name)
  beam_norm_residual_norm
                        the residual add and next norm on their own (second step
                        of the page's unfused strategy)
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_finalize.so")

MF_OK = 0
MF_DTYPE_BF16 = 1
MF_DTYPE_FP32 = 2

__all__ = ["moe_finalize_rmsnorm", "moe_finalize", "beam_moe_finalize", "mf_rmsnorm",
           "beam_moe_finalize_norm_residual_norm", "beam_norm_residual_norm",
           "FinalizeError", "lib", "LIB_PATH"]


class FinalizeError(ValueError):
    """A finalize entry point rejected its arguments or failed to launch."""

    def __init__(self, name: str, status: int, message: str):
        super().__init__(f"{name}: {message} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; build it with "
            "`python moe_expert_output_finalize_amd/build.py` (or __graft_entry__.build())")
    so = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    so.moe_finalize_rmsnorm.argtypes = [vp, i64, i64, vp, i32, vp, vp, vp, i64, i32, i32,
                                        f32, f32, i32, vp]
    so.moe_finalize.argtypes = [vp, i64, i64, vp, i32, vp, vp, i64, i32, i32, vp]
    so.beam_moe_finalize.argtypes = [vp, i64, i32, i32, vp, i64, vp, i64, vp, f32, f32, i32, vp]
    so.mf_rmsnorm.argtypes = [vp, i64, vp, vp, i64, i32, f32, f32, i32, vp]
    so.beam_moe_finalize_norm_residual_norm.argtypes = [
        vp, i64, i32, i32, vp, i64, vp, vp, vp, vp, vp, i64, f32, f32, f32, f32, f32, i32, i32, vp]
    so.beam_norm_residual_norm.argtypes = [vp, i64, vp, vp, vp, vp, vp, i64, i32, f32, f32, f32,
                                           f32, i32, i32, vp]
    for f in (so.moe_finalize_rmsnorm, so.moe_finalize, so.beam_moe_finalize, so.mf_rmsnorm,
              so.beam_moe_finalize_norm_residual_norm, so.beam_norm_residual_norm):
        f.restype = i32
    so.mf_status_string.argtypes = [ctypes.c_int]
    so.mf_status_string.restype = ctypes.c_char_p
    so.mf_last_error_message.argtypes = []
    so.mf_last_error_message.restype = ctypes.c_char_p
    return so


lib = _load()


def _raise_on(name: str, rc: int) -> None:
    if rc != MF_OK:
        msg = lib.mf_status_string(rc).decode()
        extra = lib.mf_last_error_message().decode()
        raise FinalizeError(name, rc, msg + (f": {extra}" if extra else ""))


# The current stream's raw handle without building a Stream object (torch's
# own kernel launchers use the same call); the public route costs ~2 us a call.
_current_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device: int) -> int | None:
    if stream is None:
        if _current_raw_stream is not None:
            return _current_raw_stream(device)
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _require(cond: bool, name: str, what: str) -> None:
    if not cond:
        raise ValueError(f"{name}: {what}")


def _check_device(name: str, *tensors) -> int:
    """Index of the one GPU that holds every given tensor (None entries skipped)."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        d = t.get_device()
        _require(d >= 0, name, "tensors must be on a GPU")
        if dev is None:
            dev = d
        _require(d == dev, name, "tensors must be on one device")
    return dev


def _weights_dtype(name: str, w: torch.Tensor) -> int:
    if w.dtype == torch.bfloat16:
        return MF_DTYPE_BF16
    if w.dtype == torch.float32:
        return MF_DTYPE_FP32
    raise ValueError(f"{name}: expert_weights must be bfloat16 or float32")


def _index_map_args(name, gemm2_permuted, expert_weights, idx, output):
    gshape, ishape, oshape = gemm2_permuted.shape, idx.shape, output.shape
    _require(len(gshape) == 2 and gemm2_permuted.dtype == torch.bfloat16, name,
             "gemm2_permuted must be a 2-D bfloat16 tensor")
    gstride = gemm2_permuted.stride()
    _require(gstride[1] == 1 or gshape[1] <= 1, name,
             "gemm2_permuted must have a unit-stride last dimension")
    _require(len(ishape) == 2 and idx.dtype == torch.int32 and idx.is_contiguous(), name,
             "expanded_idx_to_permuted_idx must be a contiguous int32 [tokens, top_k] tensor")
    _require(expert_weights.shape == ishape and expert_weights.is_contiguous(), name,
             "expert_weights must be contiguous with the index map's shape")
    _require(len(oshape) == 2 and output.dtype == torch.bfloat16 and output.is_contiguous(),
             name, "output must be a contiguous bfloat16 [tokens, hidden] tensor")
    _require(oshape[0] == ishape[0], name, "output and index map disagree on tokens")
    _require(gshape[1] >= oshape[1], name, "gemm2_permuted is narrower than hidden")
    row_stride = gstride[0] if gshape[0] > 1 else gshape[1]
    return (gemm2_permuted.data_ptr(), gshape[0], row_stride,
            expert_weights.data_ptr(), _weights_dtype(name, expert_weights), idx.data_ptr())


def moe_finalize_rmsnorm(gemm2_permuted: torch.Tensor, expert_weights: torch.Tensor,
                         expanded_idx_to_permuted_idx: torch.Tensor, norm_weight: torch.Tensor,
                         output: torch.Tensor, *, eps: float, gain_center: float,
                         weight_before_norm: bool, stream=None) -> None:
    """Index-map finalize fused with per-token RMSNorm, written into ``output``."""
    name = "moe_finalize_rmsnorm"
    dev = _check_device(name, gemm2_permuted, expert_weights, expanded_idx_to_permuted_idx,
                        norm_weight, output)
    g, rows, stride, w, wdt, idx = _index_map_args(name, gemm2_permuted, expert_weights,
                                                    expanded_idx_to_permuted_idx, output)
    _require(norm_weight.dim() == 1 and norm_weight.dtype == torch.bfloat16 and
             norm_weight.is_contiguous() and norm_weight.shape[0] == output.shape[1], name,
             "norm_weight must be a contiguous bfloat16 [hidden] tensor")
    T, K = expanded_idx_to_permuted_idx.shape
    rc = lib.moe_finalize_rmsnorm(g, rows, stride, w, wdt, idx, norm_weight.data_ptr(),
                                  output.data_ptr(), T, output.shape[1], K, float(eps),
                                  float(gain_center), int(bool(weight_before_norm)),
                                  _stream(stream, dev))
    _raise_on(name, rc)


def moe_finalize(gemm2_permuted: torch.Tensor, expert_weights: torch.Tensor,
                 expanded_idx_to_permuted_idx: torch.Tensor, output: torch.Tensor,
                 stream=None) -> None:
    """Index-map finalize without a norm: output = bf16(FP32 routed sum)."""
    name = "moe_finalize"
    dev = _check_device(name, gemm2_permuted, expert_weights, expanded_idx_to_permuted_idx,
                        output)
    g, rows, stride, w, wdt, idx = _index_map_args(name, gemm2_permuted, expert_weights,
                                                    expanded_idx_to_permuted_idx, output)
    T, K = expanded_idx_to_permuted_idx.shape
    rc = lib.moe_finalize(g, rows, stride, w, wdt, idx, output.data_ptr(), T, output.shape[1],
                          K, _stream(stream, dev))
    _raise_on(name, rc)


def beam_moe_finalize(expert_outputs: torch.Tensor, expert_weights: torch.Tensor,
                      output: torch.Tensor, routed_scale: float = 1.0,
                      post_weight: torch.Tensor | None = None, post_eps: float | None = None,
                      stream=None) -> torch.Tensor:
    """Token-major finalize of output.shape[0] live rows; returns ``output``."""
    name = "beam_moe_finalize"
    dev = _check_device(name, expert_outputs, expert_weights, output, post_weight)
    _require(expert_outputs.dim() == 3 and expert_weights.dim() == 2 and output.dim() == 2,
             name, "expected [capacity, top_k, hidden], [rows, top_k] and [live, hidden]")
    capacity, top_k, hidden = expert_outputs.shape
    _require(expert_outputs.dtype == torch.bfloat16 and output.dtype == torch.bfloat16, name,
             "expert_outputs and output must be bfloat16")
    _require(expert_weights.dtype == torch.float32, name, "expert_weights must be float32")
    for t in (expert_outputs, expert_weights, output):
        _require(t.is_contiguous(), name, "tensors must be contiguous")
    _require(output.shape[1] == hidden and expert_weights.shape[1] == top_k, name,
             "hidden / top_k mismatch")
    if post_weight is not None:
        _require(post_eps is not None, name, "post_weight needs post_eps")
        _require(post_weight.shape == (hidden,) and post_weight.dtype == torch.bfloat16 and
                 post_weight.is_contiguous(), name,
                 "post_weight must be a contiguous bfloat16 [hidden] tensor")
    rc = lib.beam_moe_finalize(
        expert_outputs.data_ptr(), capacity, top_k, hidden, expert_weights.data_ptr(),
        expert_weights.shape[0], output.data_ptr(), output.shape[0],
        None if post_weight is None else post_weight.data_ptr(), float(routed_scale),
        float(post_eps or 0.0), int(post_eps is not None), _stream(stream, dev))
    _raise_on(name, rc)
    return output


def mf_rmsnorm(input: torch.Tensor, norm_weight: torch.Tensor, output: torch.Tensor, *,
               eps: float, gain_center: float, weight_before_norm: bool, stream=None) -> None:
    """Standalone per-token RMSNorm of BF16 rows, written into ``output``."""
    name = "mf_rmsnorm"
    dev = _check_device(name, input, norm_weight, output)
    _require(input.dim() == 2 and input.dtype == torch.bfloat16 and
             (input.stride(1) == 1 or input.shape[1] <= 1), name,
             "input must be a 2-D bfloat16 tensor with a unit-stride last dimension")
    _require(output.dim() == 2 and output.dtype == torch.bfloat16 and output.is_contiguous() and
             output.shape[0] == input.shape[0] and input.shape[1] >= output.shape[1], name,
             "output must be a contiguous bfloat16 [tokens, hidden] tensor")
    _require(norm_weight.dim() == 1 and norm_weight.dtype == torch.bfloat16 and
             norm_weight.is_contiguous() and norm_weight.shape[0] == output.shape[1], name,
             "norm_weight must be a contiguous bfloat16 [hidden] tensor")
    stride = input.stride(0) if input.shape[0] > 1 else input.shape[1]
    rc = lib.mf_rmsnorm(input.data_ptr(), stride, norm_weight.data_ptr(), output.data_ptr(),
                        output.shape[0], output.shape[1], float(eps), float(gain_center),
                        int(bool(weight_before_norm)), _stream(stream, dev))
    _raise_on(name, rc)


def _opt_ptr(t):
    return None if t is None else t.data_ptr()


def _outputs(name, residual, next_eps, hidden_out, normalized_out):
    """(hidden, normalized) destinations: the given tensors, or new ones."""
    def ok(t):
        return (t.shape == residual.shape and t.dtype == torch.bfloat16 and t.is_contiguous()
                and t.device == residual.device)
    if hidden_out is None:
        hidden_out = torch.empty_like(residual)
    _require(ok(hidden_out), name, "hidden_out must be a contiguous bfloat16 tensor like residual")
    if next_eps is None:
        return hidden_out, None
    if normalized_out is None:
        normalized_out = torch.empty_like(residual)
    _require(ok(normalized_out), name,
             "normalized_out must be a contiguous bfloat16 tensor like residual")
    return hidden_out, normalized_out


def _check_norm_weight(name, w, eps, hidden, what):
    if w is None:
        return
    _require(eps is not None, name, f"{what} needs its eps")
    _require(w.shape == (hidden,) and w.dtype == torch.bfloat16 and w.is_contiguous(), name,
             f"{what} must be a contiguous bfloat16 [hidden] tensor")


def beam_moe_finalize_norm_residual_norm(
        expert_outputs: torch.Tensor, expert_weights: torch.Tensor, residual: torch.Tensor,
        post_weight: torch.Tensor | None, post_eps: float | None,
        next_weight: torch.Tensor | None, next_eps: float | None,
        scales: tuple[float, float] | None, routed_scale: float = 1.0, stream=None, *,
        hidden_out: torch.Tensor | None = None, normalized_out: torch.Tensor | None = None):
    """Fused token-major finalize -> (post-norm) -> residual add -> next norm
    for residual.shape[0] tokens; returns (hidden, normalized or None).

    ``expert_outputs`` is [capacity, top_k, hidden] (the producer's
    [capacity * top_k, hidden] rows viewed per token).  ``hidden_out`` and
    ``normalized_out`` may be given to write into existing tensors."""
    name = "beam_moe_finalize_norm_residual_norm"
    dev = _check_device(name, expert_outputs, expert_weights, residual, post_weight,
                        next_weight)
    _require(expert_outputs.dim() == 3 and expert_weights.dim() == 2 and residual.dim() == 2,
             name, "expected [capacity, top_k, hidden], [rows, top_k] and [tokens, hidden]")
    capacity, top_k, hidden = expert_outputs.shape
    _require(expert_outputs.dtype == torch.bfloat16 and residual.dtype == torch.bfloat16,
             name, "expert_outputs and residual must be bfloat16")
    _require(expert_weights.dtype == torch.float32, name, "expert_weights must be float32")
    for t in (expert_outputs, expert_weights, residual):
        _require(t.is_contiguous(), name, "tensors must be contiguous")
    _require(residual.shape[1] == hidden and expert_weights.shape[1] == top_k, name,
             "hidden / top_k mismatch")
    _check_norm_weight(name, post_weight, post_eps, hidden, "post_weight")
    _check_norm_weight(name, next_weight, next_eps, hidden, "next_weight")
    out_h, out_n = _outputs(name, residual, next_eps, hidden_out, normalized_out)
    sx, sr = scales if scales is not None else (1.0, 1.0)
    rc = lib.beam_moe_finalize_norm_residual_norm(
        expert_outputs.data_ptr(), capacity, top_k, hidden, expert_weights.data_ptr(),
        expert_weights.shape[0], residual.data_ptr(), _opt_ptr(post_weight),
        _opt_ptr(next_weight), out_h.data_ptr(), _opt_ptr(out_n), residual.shape[0],
        float(routed_scale), float(post_eps or 0.0), float(next_eps or 0.0), float(sx),
        float(sr), int(post_eps is not None), int(next_eps is not None), _stream(stream, dev))
    _raise_on(name, rc)
    return out_h, out_n


def beam_norm_residual_norm(x: torch.Tensor, residual: torch.Tensor,
                            post_weight: torch.Tensor | None, post_eps: float | None,
                            next_weight: torch.Tensor | None, next_eps: float | None,
                            scales: tuple[float, float] | None, stream=None, *,
                            hidden_out: torch.Tensor | None = None,
                            normalized_out: torch.Tensor | None = None):
    """(Post-norm) -> residual add -> next norm of BF16 rows ``x``; returns
    (hidden, normalized or None), optionally written into given tensors."""
    name = "beam_norm_residual_norm"
    dev = _check_device(name, x, residual, post_weight, next_weight)
    _require(x.dim() == 2 and residual.dim() == 2 and x.dtype == torch.bfloat16 and
             residual.dtype == torch.bfloat16, name, "x and residual must be 2-D bfloat16")
    _require(x.stride(1) == 1 or x.shape[1] <= 1, name, "x needs a unit-stride last dimension")
    _require(residual.is_contiguous() and x.shape[0] == residual.shape[0] and
             x.shape[1] >= residual.shape[1], name, "x / residual shape mismatch")
    hidden = residual.shape[1]
    _check_norm_weight(name, post_weight, post_eps, hidden, "post_weight")
    _check_norm_weight(name, next_weight, next_eps, hidden, "next_weight")
    out_h, out_n = _outputs(name, residual, next_eps, hidden_out, normalized_out)
    sx, sr = scales if scales is not None else (1.0, 1.0)
    stride = x.stride(0) if x.shape[0] > 1 else x.shape[1]
    rc = lib.beam_norm_residual_norm(
        x.data_ptr(), stride, residual.data_ptr(), _opt_ptr(post_weight), _opt_ptr(next_weight),
        out_h.data_ptr(), _opt_ptr(out_n), residual.shape[0], hidden, float(post_eps or 0.0),
        float(next_eps or 0.0), float(sx), float(sr), int(post_eps is not None),
        int(next_eps is not None), _stream(stream, dev))
    _raise_on(name, rc)
    return out_h, out_n
