"""MoE expert-output finalize for MI355X (gfx950): Python binding.

Thin ctypes layer over ``libmoe_finalize.so`` (C ABI in
``include/moe_finalize.h``).  It only marshals torch tensors into pointers,
sizes and the current HIP stream; every step of the computation runs in the
library's HIP kernels.  There is no fallback: if the library is not built,
or was built from other sources than the ones beside it, importing this
package raises.

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

The binding checks what the C ABI cannot see (dtype, device, contiguity and
that the tensors' shapes agree) and hands every size to the library, which
enforces the value ranges (top-k, hidden, live rows against capacity and
weight rows, optional weights only with their norm) and returns a status
that becomes a ``FinalizeError`` (a ``ValueError``).
"""
from __future__ import annotations

import ctypes
import importlib.util
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


def _build_module():
    spec = importlib.util.spec_from_file_location("_mf_build", os.path.join(_PKG, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def check_built(lib_path: str = LIB_PATH) -> None:
    """Raise ImportError unless `lib_path` exists and was built from the
    sources now beside it (the digest its build recorded matches)."""
    how = ("build it with `python moe_expert_output_finalize_amd/build.py` "
           "(or __graft_entry__.build())")
    if not os.path.exists(lib_path):
        raise ImportError(f"{lib_path} is not built; {how}")
    b = _build_module()
    try:
        with open(b.digest_path(lib_path)) as f:
            recorded = f.read().strip()
    except OSError:
        raise ImportError(f"{lib_path} has no record of its sources; rebuild: {how}") from None
    root = os.path.dirname(os.path.dirname(os.path.abspath(lib_path)))
    if recorded != b.source_digest(root):
        raise ImportError(f"{lib_path} was built from other sources than the ones beside it "
                          f"(stale or a variant build); rebuild: {how}")


def _load() -> ctypes.CDLL:
    check_built()
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


# ------------------------------------------------------------ checks -------
#
# These run on every call, so each tensor's attributes are read once and an
# error message is only built for a failed check.

def _fail(name: str, what: str):
    raise ValueError(f"{name}: {what}")


def _t(name: str, what: str, t, dtype, ndim: int, contiguous: bool = True):
    """Shape of `t` after checking its dtype, rank and layout (contiguous, or
    unit stride along the last dimension only)."""
    if t is None:
        _fail(name, f"{what} is required")
    shape = t.shape
    if (t.dtype is not dtype or len(shape) != ndim or
            not (t.is_contiguous() if contiguous else (shape[-1] <= 1 or t.stride(-1) == 1))):
        layout = "contiguous" if contiguous else "unit-stride rows"
        _fail(name, f"{what} must be a {ndim}-D {layout} {dtype} tensor, got {t.dtype} "
                    f"{tuple(shape)} with strides {t.stride()}")
    return shape


def _device(name: str, *tensors) -> int:
    """Index of the one GPU that holds every given tensor (None entries skipped)."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        d = t.get_device()
        if d < 0 or (dev is not None and d != dev):
            _fail(name, "tensors must be on one GPU")
        dev = d
    return dev


def _vector(name: str, what: str, t, hidden: int) -> int | None:
    """Pointer of an optional BF16 [hidden] weight (None stays None)."""
    if t is None:
        return None
    if _t(name, what, t, torch.bfloat16, 1)[0] != hidden:
        _fail(name, f"{what} must have {hidden} elements")
    return t.data_ptr()


def _row_stride(t, shape) -> int:
    """Elements between the rows of a 2-D tensor with unit-stride rows."""
    return t.stride(0) if shape[0] > 1 else shape[1]


def _weights_dtype(name: str, w: torch.Tensor) -> int:
    d = w.dtype
    if d is torch.float32:
        return MF_DTYPE_FP32
    if d is torch.bfloat16:
        return MF_DTYPE_BF16
    _fail(name, "expert_weights must be bfloat16 or float32")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _eps(eps) -> tuple[float, int]:
    """An optional epsilon as the C ABI's (value, present) pair."""
    return (0.0, 0) if eps is None else (float(eps), 1)


# ------------------------------------------------- index-map entry points --
#
# FlashInfer "flashinfer.comm.tp_moe_finalize_rmsnorm", Parameters:
# gemm2_permuted BF16 [rows, >= hidden] with unit-stride rows; expert_weights
# BF16 or FP32 [tokens, top_k] and expanded_idx_to_permuted_idx int32
# [tokens, top_k], both contiguous; norm_weight BF16 [hidden]; output BF16
# [tokens, hidden], contiguous.

def _index_map(name, gemm2_permuted, expert_weights, idx, output):
    T, K = _t(name, "expanded_idx_to_permuted_idx", idx, torch.int32, 2)
    wdt = _weights_dtype(name, expert_weights)
    if _t(name, "expert_weights", expert_weights, expert_weights.dtype, 2) != (T, K):
        _fail(name, "expert_weights must have the index map's shape")
    To, H = _t(name, "output", output, torch.bfloat16, 2)
    gshape = _t(name, "gemm2_permuted", gemm2_permuted, torch.bfloat16, 2, contiguous=False)
    if To != T or gshape[1] < H:
        _fail(name, "output must be [tokens, hidden] and gemm2_permuted at least hidden wide")
    return (gemm2_permuted.data_ptr(), gshape[0], _row_stride(gemm2_permuted, gshape),
            expert_weights.data_ptr(), wdt, idx.data_ptr(), T, H, K)


def moe_finalize_rmsnorm(gemm2_permuted: torch.Tensor, expert_weights: torch.Tensor,
                         expanded_idx_to_permuted_idx: torch.Tensor, norm_weight: torch.Tensor,
                         output: torch.Tensor, *, eps: float, gain_center: float,
                         weight_before_norm: bool, stream=None) -> None:
    """Index-map finalize fused with per-token RMSNorm, written into ``output``."""
    name = "moe_finalize_rmsnorm"
    dev = _device(name, gemm2_permuted, expert_weights, expanded_idx_to_permuted_idx,
                  norm_weight, output)
    g, rows, stride, w, wdt, idx, T, H, K = _index_map(
        name, gemm2_permuted, expert_weights, expanded_idx_to_permuted_idx, output)
    nw = _vector(name, "norm_weight", norm_weight, H)
    if nw is None:
        _fail(name, "norm_weight is required")
    rc = lib.moe_finalize_rmsnorm(g, rows, stride, w, wdt, idx, nw, output.data_ptr(), T, H, K,
                                  float(eps), float(gain_center), int(bool(weight_before_norm)),
                                  _stream(stream, dev))
    if rc:
        _raise_on(name, rc)


def moe_finalize(gemm2_permuted: torch.Tensor, expert_weights: torch.Tensor,
                 expanded_idx_to_permuted_idx: torch.Tensor, output: torch.Tensor,
                 stream=None) -> None:
    """Index-map finalize without a norm: output = bf16(FP32 routed sum)."""
    name = "moe_finalize"
    dev = _device(name, gemm2_permuted, expert_weights, expanded_idx_to_permuted_idx, output)
    g, rows, stride, w, wdt, idx, T, H, K = _index_map(
        name, gemm2_permuted, expert_weights, expanded_idx_to_permuted_idx, output)
    rc = lib.moe_finalize(g, rows, stride, w, wdt, idx, output.data_ptr(), T, H, K,
                          _stream(stream, dev))
    if rc:
        _raise_on(name, rc)


def mf_rmsnorm(input: torch.Tensor, norm_weight: torch.Tensor, output: torch.Tensor, *,
               eps: float, gain_center: float, weight_before_norm: bool, stream=None) -> None:
    """Standalone per-token RMSNorm of BF16 rows, written into ``output``."""
    name = "mf_rmsnorm"
    dev = _device(name, input, norm_weight, output)
    T, H = _t(name, "output", output, torch.bfloat16, 2)
    ishape = _t(name, "input", input, torch.bfloat16, 2, contiguous=False)
    if ishape[0] != T or ishape[1] < H:
        _fail(name, "input must have output's rows and be at least as wide")
    nw = _vector(name, "norm_weight", norm_weight, H)
    if nw is None:
        _fail(name, "norm_weight is required")
    rc = lib.mf_rmsnorm(input.data_ptr(), _row_stride(input, ishape), nw, output.data_ptr(), T,
                        H, float(eps), float(gain_center), int(bool(weight_before_norm)),
                        _stream(stream, dev))
    if rc:
        _raise_on(name, rc)


# ----------------------------------------------- token-major entry points --
#
# vLLM "vllm.models.beam.nvidia.moe_finalize", Parameters of
# beam_moe_finalize: expert_outputs contiguous BF16 [capacity, top_k, hidden];
# expert_weights contiguous FP32 with top_k columns and a row per token slot;
# the per-token destination (and, for the residual variants, the residual)
# contiguous BF16 [tokens, hidden]; optional BF16 norm weights [hidden], each
# used only when its epsilon is given.

def _token_major(name, expert_outputs, expert_weights, per_token, what):
    capacity, top_k, hidden = _t(name, "expert_outputs", expert_outputs, torch.bfloat16, 3)
    wshape = _t(name, "expert_weights", expert_weights, torch.float32, 2)
    pshape = _t(name, what, per_token, torch.bfloat16, 2)
    if wshape[1] != top_k or pshape[1] != hidden:
        _fail(name, f"expert_weights must have top_k columns and {what} hidden columns")
    return capacity, top_k, hidden, wshape[0], pshape[0]


def beam_moe_finalize(expert_outputs: torch.Tensor, expert_weights: torch.Tensor,
                      output: torch.Tensor, routed_scale: float = 1.0,
                      post_weight: torch.Tensor | None = None, post_eps: float | None = None,
                      stream=None) -> torch.Tensor:
    """Token-major finalize of output.shape[0] live rows; returns ``output``."""
    name = "beam_moe_finalize"
    dev = _device(name, expert_outputs, expert_weights, output, post_weight)
    capacity, top_k, hidden, wrows, live = _token_major(name, expert_outputs, expert_weights,
                                                        output, "output")
    pw = _vector(name, "post_weight", post_weight, hidden)
    eps, has_norm = _eps(post_eps)
    rc = lib.beam_moe_finalize(expert_outputs.data_ptr(), capacity, top_k, hidden,
                               expert_weights.data_ptr(), wrows, output.data_ptr(), live, pw,
                               float(routed_scale), eps, has_norm, _stream(stream, dev))
    if rc:
        _raise_on(name, rc)
    return output


def _residual_outputs(name, residual, has_next, hidden_out, normalized_out):
    """(hidden, normalized) destinations: the given tensors, or new ones
    shaped like the residual."""
    shape = residual.shape
    if hidden_out is None:
        hidden_out = torch.empty_like(residual)
    elif _t(name, "hidden_out", hidden_out, torch.bfloat16, 2) != shape:
        _fail(name, "hidden_out must have the residual's shape")
    if not has_next:
        return hidden_out, None
    if normalized_out is None:
        normalized_out = torch.empty_like(residual)
    elif _t(name, "normalized_out", normalized_out, torch.bfloat16, 2) != shape:
        _fail(name, "normalized_out must have the residual's shape")
    return hidden_out, normalized_out


def _scales(scales) -> tuple[float, float]:
    """The scales pair (finalized branch, residual); absent means (1, 1)."""
    sx, sr = (1.0, 1.0) if scales is None else scales
    return float(sx), float(sr)


def beam_moe_finalize_norm_residual_norm(
        expert_outputs: torch.Tensor, expert_weights: torch.Tensor, residual: torch.Tensor,
        post_weight: torch.Tensor | None, post_eps: float | None,
        next_weight: torch.Tensor | None, next_eps: float | None,
        scales: tuple[float, float] | None, routed_scale: float = 1.0, stream=None, *,
        hidden_out: torch.Tensor | None = None, normalized_out: torch.Tensor | None = None,
        strategy: str | None = None):
    """Fused token-major finalize -> (post-norm) -> residual add -> next norm
    for residual.shape[0] tokens; returns (hidden, normalized or None).

    ``expert_outputs`` is [capacity, top_k, hidden] (the producer's
    [capacity * top_k, hidden] rows viewed per token).  ``hidden_out`` and
    ``normalized_out`` may be given to write into existing tensors.
    ``strategy`` (the page's keyword of the same name, "vllm.models.beam.
    nvidia.moe_finalize"): None or "fused" runs the fused kernel; "unfused"
    runs beam_moe_finalize into a BF16 intermediate and then
    beam_norm_residual_norm, the two-step reference kept for validation and
    benchmarking (bit-identical results); anything else raises ValueError."""
    name = "beam_moe_finalize_norm_residual_norm"
    if strategy not in (None, "fused", "unfused"):
        raise ValueError(f"{name}: unknown strategy {strategy!r} (None, 'fused' or 'unfused')")
    if strategy == "unfused":
        T, hidden = _t(name, "residual", residual, torch.bfloat16, 2)
        y = torch.empty((T, hidden), dtype=torch.bfloat16, device=residual.device)
        beam_moe_finalize(expert_outputs, expert_weights, y, routed_scale, post_weight,
                          post_eps, stream)
        return beam_norm_residual_norm(y, residual, None, None, next_weight, next_eps, scales,
                                       stream, hidden_out=hidden_out,
                                       normalized_out=normalized_out)
    dev = _device(name, expert_outputs, expert_weights, residual, post_weight, next_weight,
                  hidden_out, normalized_out)
    capacity, top_k, hidden, wrows, T = _token_major(name, expert_outputs, expert_weights,
                                                     residual, "residual")
    pw = _vector(name, "post_weight", post_weight, hidden)
    nw = _vector(name, "next_weight", next_weight, hidden)
    peps, has_post = _eps(post_eps)
    neps, has_next = _eps(next_eps)
    out_h, out_n = _residual_outputs(name, residual, has_next, hidden_out, normalized_out)
    sx, sr = _scales(scales)
    rc = lib.beam_moe_finalize_norm_residual_norm(
        expert_outputs.data_ptr(), capacity, top_k, hidden, expert_weights.data_ptr(), wrows,
        residual.data_ptr(), pw, nw, out_h.data_ptr(), _ptr(out_n), T, float(routed_scale),
        peps, neps, sx, sr, has_post, has_next, _stream(stream, dev))
    if rc:
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
    dev = _device(name, x, residual, post_weight, next_weight, hidden_out, normalized_out)
    T, hidden = _t(name, "residual", residual, torch.bfloat16, 2)
    xshape = _t(name, "x", x, torch.bfloat16, 2, contiguous=False)
    if xshape[0] != T or xshape[1] < hidden:
        _fail(name, "x must have the residual's rows and be at least as wide")
    pw = _vector(name, "post_weight", post_weight, hidden)
    nw = _vector(name, "next_weight", next_weight, hidden)
    peps, has_post = _eps(post_eps)
    neps, has_next = _eps(next_eps)
    out_h, out_n = _residual_outputs(name, residual, has_next, hidden_out, normalized_out)
    sx, sr = _scales(scales)
    rc = lib.beam_norm_residual_norm(
        x.data_ptr(), _row_stride(x, xshape), residual.data_ptr(), pw, nw, out_h.data_ptr(),
        _ptr(out_n), T, hidden, peps, neps, sx, sr, has_post, has_next, _stream(stream, dev))
    if rc:
        _raise_on(name, rc)
    return out_h, out_n
