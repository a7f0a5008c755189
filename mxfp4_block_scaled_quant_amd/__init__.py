"""W4A4 MXFP4 linear and A16WFP4 batched GEMM for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libmxfp4.so`` (C ABI in ``include/mxfp4.h``).
Every step of the computation runs in the library's HIP kernels; this module
only allocates output tensors with torch, passes raw device pointers and the
current HIP stream, and turns status codes into exceptions.  There is no
fallback: if the library is missing or the device is not gfx950, calls fail.

Entry points (same names as the C ABI):

* :func:`mxfp4_quant_1x32` -- bf16 [M, K] -> packed FP4 [M, K/2] + E8M0 scales
* :func:`mxfp4_preshuffle_weight` -- quantised weights -> preshuffled layout
* :func:`mxfp4_gemm_a4w4` -- W4A4 GEMM with optional bias, bf16/fp32 out
* :func:`mxfp4_linear` -- bf16 activations -> quant + GEMM (+ bias) in one call,
  the quantisation fused into the GEMM kernel (one launch) at M = 1, at
  M = 2 up to K = 16384, at M <= 4 where N < 16384 and K <= 8192 (but not
  3-4 rows at 8192 < N <= 12288) or N <= 4096 and K <= 16384, and at
  2 <= M <= 4 on wide N with 4608 < K <= 6144; otherwise quantised into a
  workspace first (two launches)
* :func:`mxfp4_gemm_a4w4_mxfp4_out` -- the GEMM writing MXFP4 (row-major FP4 +
  E8M0) for the next layer
* :func:`mxfp4_shuffle_scales` -- row-major E8M0 scales -> the GEMM scale layout
* :func:`mxfp4_linear_prequantized` -- the linear from row-major packed FP4 +
  scales handed over by a producer
* :func:`a16wfp4_bmm` -- bf16 [B, M, K] x MXFP4 [B, N, K] batched GEMM

Convenience: :func:`quantize_weight` (quant + preshuffle, once at load) and
:func:`linear` (:func:`mxfp4_linear` over any leading dimensions).  The same
entry points as torch custom operators (``torch.ops.mxfp4.*``, with fake
implementations for tracing and torch.compile) are registered by importing
:mod:`mxfp4_block_scaled_quant_amd.ops`.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmxfp4.so")

MXFP4_LAYOUT_ROWMAJOR = 0
MXFP4_LAYOUT_GEMM = 1
MXFP4_OUT_BF16 = 0
MXFP4_OUT_F32 = 1

_c_i64 = ctypes.c_int64
_c_vp = ctypes.c_void_p
_c_int = ctypes.c_int
_c_size = ctypes.c_size_t

_SIGNATURES = {
    "mxfp4_status_str": (ctypes.c_char_p, [_c_int]),
    "mxfp4_abi_version": (_c_int, []),
    "mxfp4_data_bytes": (_c_size, [_c_i64, _c_i64, _c_int]),
    "mxfp4_scale_bytes": (_c_size, [_c_i64, _c_i64, _c_int]),
    "mxfp4_weight_bytes": (_c_size, [_c_i64, _c_i64, _c_i64]),
    "mxfp4_weight_scale_bytes": (_c_size, [_c_i64, _c_i64, _c_i64]),
    "mxfp4_gemm_workspace_bytes": (_c_size, [_c_i64, _c_i64, _c_i64]),
    "mxfp4_quant_1x32": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_i64, _c_vp, _c_int, _c_vp]),
    "mxfp4_preshuffle_weight": (_c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp]),
    "mxfp4_gemm_a4w4": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_int,
                                 _c_i64, _c_i64, _c_i64, _c_vp, _c_size, _c_vp]),
    "mxfp4_linear_workspace_bytes": (_c_size, [_c_i64, _c_i64, _c_i64]),
    "mxfp4_linear": (_c_int, [_c_vp, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_int,
                              _c_i64, _c_i64, _c_i64, _c_vp, _c_size, _c_vp]),
    "mxfp4_linear_noalloc": (_c_int, [_c_vp, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_int,
                                      _c_i64, _c_i64, _c_i64, _c_vp]),
    "mxfp4_gemm_a4w4_mxfp4_out": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_vp,
                                           _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_size, _c_vp]),
    "mxfp4_shuffle_scales": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp]),
    "mxfp4_linear_prequantized_workspace_bytes": (_c_size, [_c_i64, _c_i64, _c_i64]),
    "mxfp4_linear_prequantized": (_c_int, [_c_vp, _c_i64, _c_vp, _c_i64, _c_vp, _c_vp, _c_vp,
                                           _c_vp, _c_i64, _c_int, _c_i64, _c_i64, _c_i64,
                                           _c_vp, _c_size, _c_vp]),
    "a16wfp4_bmm": (_c_int, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_int,
                             _c_i64, _c_i64, _c_i64, _c_i64, _c_vp]),
    "mxfp4_testing_set_gemm_path": (_c_int, [_c_int]),
}

_lib_handle = None


class MXFP4Error(RuntimeError):
    """A libmxfp4 call returned a non-zero status."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libmxfp4.so (built in place by ``python -m mxfp4_block_scaled_quant_amd.build``)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mxfp4_block_scaled_quant_amd.build` (hipcc, gfx950)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib_handle = h
    return _lib_handle


def _check(fn: str, status: int) -> None:
    if status != 0:
        msg = lib().mxfp4_status_str(status).decode()
        raise MXFP4Error(fn, status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require_cuda(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (cuda/HIP) tensor")


def _require_bytes(t: Optional[torch.Tensor], name: str, nbytes: int, device: torch.device) -> None:
    """t is a uint8 tensor on `device`, contiguous, of at least nbytes bytes."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != torch.uint8 or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous uint8 tensor on {device}")
    if t.numel() < nbytes:
        raise ValueError(f"{name} holds {t.numel()} bytes, {nbytes} needed")


def _require_out(out: torch.Tensor, shape, dtype: torch.dtype, device: torch.device) -> None:
    """A caller's output: this shape and dtype on `device`, unit stride along
    its last dimension (the kernels write whole rows from there)."""
    if tuple(out.shape) != tuple(shape) or out.dtype != dtype or out.device != device:
        raise ValueError(f"out must be {tuple(shape)} {dtype} on {device}, "
                         f"got {tuple(out.shape)} {out.dtype} on {out.device}")
    if out.numel() and out.stride(-1) != 1:
        raise ValueError("out must have unit stride along its last dimension")


def _require_bias(bias: Optional[torch.Tensor], N: int, device: torch.device) -> None:
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() != N
                             or bias.device != device or not bias.is_contiguous()):
        raise ValueError(f"bias must be a contiguous bf16 [N = {N}] tensor on {device}")


def _require_weight(w_pre: torch.Tensor, ws_pre: torch.Tensor, N: int, K: int,
                    device: torch.device, batch: int = 1) -> None:
    _require_bytes(w_pre, "w_pre", weight_bytes(batch, N, K), device)
    _require_bytes(ws_pre, "ws_pre", weight_scale_bytes(batch, N, K), device)


def data_bytes(rows: int, K: int, layout: int) -> int:
    return int(lib().mxfp4_data_bytes(rows, K, layout))


def scale_bytes(rows: int, K: int, layout: int) -> int:
    return int(lib().mxfp4_scale_bytes(rows, K, layout))


def weight_bytes(batch: int, N: int, K: int) -> int:
    return int(lib().mxfp4_weight_bytes(batch, N, K))


def weight_scale_bytes(batch: int, N: int, K: int) -> int:
    return int(lib().mxfp4_weight_scale_bytes(batch, N, K))


def set_gemm_path(path: int) -> None:
    """Test hook (include/mxfp4_testing.h), for the calling thread only: 1
    forces the small-M kernel (M <= 64), 2 the tiled kernel, 0 = by M and N
    (the small-M kernel up to 64 rows, and once per 64 rows up to 256 rows
    where ceil(M/64) * N <= 16384); 3 the
    tiled kernel on whole 256-wide tiles only, 4 with the split (split-K)
    schedule; 5 and 6 the same with 128-wide tiles."""
    _check("mxfp4_testing_set_gemm_path", lib().mxfp4_testing_set_gemm_path(path))


def mxfp4_quant_1x32(x: torch.Tensor, layout: int = MXFP4_LAYOUT_GEMM,
                     q: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None):
    """Quantise bf16 rows [M, K] per 1x32 block.  Returns (q, scales) uint8 tensors.

    MXFP4_LAYOUT_GEMM (default): both 1-D in the GEMM layouts (what
    :func:`mxfp4_gemm_a4w4` reads).  MXFP4_LAYOUT_ROWMAJOR: q [M, K/2] (any
    row stride) and scales [M*K/32].
    """
    _require_cuda(x, "x")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit stride along K")
    M, K = x.shape
    if q is None:
        if layout == MXFP4_LAYOUT_ROWMAJOR:
            q = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
        else:
            q = torch.empty(data_bytes(M, K, layout), dtype=torch.uint8, device=x.device)
    elif layout == MXFP4_LAYOUT_ROWMAJOR and q.dim() == 2:
        if q.dtype != torch.uint8 or q.device != x.device or q.shape != (M, K // 2) or q.stride(1) != 1:
            raise ValueError(f"q must be uint8 [{M}, {K // 2}] with unit stride along K on {x.device}")
    else:
        _require_bytes(q, "q", data_bytes(M, K, layout), x.device)
    if scales is None:
        scales = torch.empty(scale_bytes(M, K, layout), dtype=torch.uint8, device=x.device)
    else:
        _require_bytes(scales, "scales", scale_bytes(M, K, layout), x.device)
    ldq = q.stride(0) if (layout == MXFP4_LAYOUT_ROWMAJOR and q.dim() == 2) else K // 2
    _check("mxfp4_quant_1x32", lib().mxfp4_quant_1x32(
        _ptr(x), M, K, x.stride(0), _ptr(q), ldq, _ptr(scales), layout, _stream(x.device)))
    return q, scales


def mxfp4_preshuffle_weight(w_fp4: torch.Tensor, w_scales: torch.Tensor, N: int, K: int,
                            batch: int = 1):
    """Row-major packed FP4 weights + row-major scales -> (w_pre, ws_pre) uint8 1-D."""
    _require_cuda(w_fp4, "w_fp4")
    if not (w_fp4.is_contiguous() and w_scales.is_contiguous()):
        raise ValueError("w_fp4 and w_scales must be contiguous")
    if w_fp4.numel() != batch * N * K // 2 or w_scales.numel() != batch * N * K // 32:
        raise ValueError("w_fp4 / w_scales sizes do not match (batch, N, K)")
    w_pre = torch.empty(weight_bytes(batch, N, K), dtype=torch.uint8, device=w_fp4.device)
    ws_pre = torch.empty(weight_scale_bytes(batch, N, K), dtype=torch.uint8, device=w_fp4.device)
    _check("mxfp4_preshuffle_weight", lib().mxfp4_preshuffle_weight(
        _ptr(w_fp4), _ptr(w_scales), batch, N, K, _ptr(w_pre), _ptr(ws_pre), _stream(w_fp4.device)))
    return w_pre, ws_pre


def gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().mxfp4_gemm_workspace_bytes(M, N, K))


def _gemm_operands(a_fp4, a_scales, w_pre, ws_pre, M, N, K, bias):
    _require_cuda(a_fp4, "a_fp4")
    dev = a_fp4.device
    _require_bytes(a_fp4, "a_fp4", data_bytes(M, K, MXFP4_LAYOUT_GEMM), dev)
    _require_bytes(a_scales, "a_scales", scale_bytes(M, K, MXFP4_LAYOUT_GEMM), dev)
    _require_weight(w_pre, ws_pre, N, K, dev)
    _require_bias(bias, N, dev)
    return dev


def _gemm_workspace(M, N, K, workspace, dev):
    need = gemm_workspace_bytes(M, N, K)
    if workspace is None:
        return (torch.empty(need, dtype=torch.uint8, device=dev) if need else None), need
    _require_bytes(workspace, "workspace", need, dev)
    return workspace, workspace.numel()


def mxfp4_gemm_a4w4(a_fp4: torch.Tensor, a_scales: torch.Tensor, w_pre: torch.Tensor,
                    ws_pre: torch.Tensor, M: int, N: int, K: int,
                    bias: Optional[torch.Tensor] = None,
                    out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None):
    """out[M, N] = dq(A) dq(W)^T (+ bias), bf16 or fp32; A and W in the GEMM layouts.

    ``workspace`` (uint8, >= :func:`gemm_workspace_bytes`) is allocated here
    when needed and not given; after a call that used one, its first 32-bit
    word is nonzero if the split schedule's bounded wait gave up."""
    dev = _gemm_operands(a_fp4, a_scales, w_pre, ws_pre, M, N, K, bias)
    code = {torch.bfloat16: MXFP4_OUT_BF16, torch.float32: MXFP4_OUT_F32}[out_dtype]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    else:
        _require_out(out, (M, N), out_dtype, dev)
    workspace, ws_bytes = _gemm_workspace(M, N, K, workspace, dev)
    _check("mxfp4_gemm_a4w4", lib().mxfp4_gemm_a4w4(
        _ptr(a_fp4), _ptr(a_scales), _ptr(w_pre), _ptr(ws_pre), _ptr(bias),
        _ptr(out), out.stride(0), code, M, N, K, _ptr(workspace), ws_bytes, _stream(a_fp4.device)))
    return out


def linear_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().mxfp4_linear_workspace_bytes(M, N, K))


def mxfp4_linear(x: torch.Tensor, w_pre: torch.Tensor, ws_pre: torch.Tensor, N: int,
                 bias: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
                 out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """out[M, N] = round(dq(Q(x)) dq(W)^T (+ bias)) from bf16 x [M, K] (unit stride along K).

    ``workspace`` (uint8, >= :func:`linear_workspace_bytes` bytes) is
    allocated here when needed and not given; the fused shapes (see the
    module docstring) need none and leave it untouched.
    """
    _require_cuda(x, "x")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit stride along K")
    M, K = x.shape
    _require_weight(w_pre, ws_pre, N, K, x.device)
    _require_bias(bias, N, x.device)
    code = {torch.bfloat16: MXFP4_OUT_BF16, torch.float32: MXFP4_OUT_F32}[out_dtype]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    else:
        _require_out(out, (M, N), out_dtype, x.device)
    need = linear_workspace_bytes(M, N, K)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    elif workspace is not None:
        _require_bytes(workspace, "workspace", need, x.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check("mxfp4_linear", lib().mxfp4_linear(
        _ptr(x), x.stride(0), _ptr(w_pre), _ptr(ws_pre), _ptr(bias), _ptr(out), out.stride(0),
        code, M, N, K, _ptr(workspace), ws_bytes, _stream(x.device)))
    return out


def mxfp4_linear_noalloc(x: torch.Tensor, w_pre: torch.Tensor, ws_pre: torch.Tensor, N: int,
                         bias: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
                         out: Optional[torch.Tensor] = None):
    """:func:`mxfp4_linear` through the entry point that allocates nothing and
    takes no workspace (the library's own per-GPU scratch holds the quantised
    activations; calls that overlap on one GPU race).  Only ``out`` is
    allocated here, and only when not given."""
    _require_cuda(x, "x")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit stride along K")
    M, K = x.shape
    _require_weight(w_pre, ws_pre, N, K, x.device)
    _require_bias(bias, N, x.device)
    code = {torch.bfloat16: MXFP4_OUT_BF16, torch.float32: MXFP4_OUT_F32}[out_dtype]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    else:
        _require_out(out, (M, N), out_dtype, x.device)
    _check("mxfp4_linear_noalloc", lib().mxfp4_linear_noalloc(
        _ptr(x), x.stride(0), _ptr(w_pre), _ptr(ws_pre), _ptr(bias), _ptr(out), out.stride(0),
        code, M, N, K, _stream(x.device)))
    return out


def mxfp4_gemm_a4w4_mxfp4_out(a_fp4: torch.Tensor, a_scales: torch.Tensor, w_pre: torch.Tensor,
                              ws_pre: torch.Tensor, M: int, N: int, K: int,
                              bias: Optional[torch.Tensor] = None,
                              out_fp4: Optional[torch.Tensor] = None,
                              out_scales: Optional[torch.Tensor] = None,
                              workspace: Optional[torch.Tensor] = None):
    """(q [M, N/2], scales [M, N/32]) uint8: the GEMM's rows quantised per 1x32
    along N (bitwise mxfp4_quant_1x32 of the bf16 output, ROWMAJOR)."""
    dev = _gemm_operands(a_fp4, a_scales, w_pre, ws_pre, M, N, K, bias)
    if out_fp4 is None:
        out_fp4 = torch.empty((M, N // 2), dtype=torch.uint8, device=dev)
    else:
        _require_out(out_fp4, (M, N // 2), torch.uint8, dev)
    if out_scales is None:
        out_scales = torch.empty((M, N // 32), dtype=torch.uint8, device=dev)
    else:
        _require_out(out_scales, (M, N // 32), torch.uint8, dev)
    workspace, ws_bytes = _gemm_workspace(M, N, K, workspace, dev)
    _check("mxfp4_gemm_a4w4_mxfp4_out", lib().mxfp4_gemm_a4w4_mxfp4_out(
        _ptr(a_fp4), _ptr(a_scales), _ptr(w_pre), _ptr(ws_pre), _ptr(bias), _ptr(out_fp4),
        out_fp4.stride(0), _ptr(out_scales), out_scales.stride(0), M, N, K, _ptr(workspace),
        ws_bytes, _stream(a_fp4.device)))
    return out_fp4, out_scales


def mxfp4_shuffle_scales(scales: torch.Tensor, rows: int, K: int,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Row-major E8M0 scales [rows, K/32] (any row stride, unit stride along
    the blocks) -> 1-D uint8 in the GEMM scale layout, padding 0x7F."""
    _require_cuda(scales, "scales")
    s2 = scales.reshape(rows, K // 32) if scales.dim() == 1 else scales
    if s2.dtype != torch.uint8 or s2.shape != (rows, K // 32) or s2.stride(1) != 1:
        raise ValueError("scales must be uint8 [rows, K/32] with unit stride along the blocks")
    if out is None:
        out = torch.empty(scale_bytes(rows, K, MXFP4_LAYOUT_GEMM), dtype=torch.uint8,
                          device=scales.device)
    else:
        _require_bytes(out, "out", scale_bytes(rows, K, MXFP4_LAYOUT_GEMM), scales.device)
    _check("mxfp4_shuffle_scales", lib().mxfp4_shuffle_scales(
        _ptr(s2), s2.stride(0), rows, K, _ptr(out), _stream(scales.device)))
    return out


def linear_prequantized_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().mxfp4_linear_prequantized_workspace_bytes(M, N, K))


def mxfp4_linear_prequantized(x_fp4: torch.Tensor, x_scales: torch.Tensor, w_pre: torch.Tensor,
                              ws_pre: torch.Tensor, N: int, bias: Optional[torch.Tensor] = None,
                              out_dtype: torch.dtype = torch.bfloat16,
                              out: Optional[torch.Tensor] = None,
                              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[M, N] from row-major packed FP4 x_fp4 [M, K/2] and E8M0 x_scales
    [M, K/32] (each with unit stride along K and any row stride)."""
    _require_cuda(x_fp4, "x_fp4")
    if x_fp4.dtype != torch.uint8 or x_fp4.dim() != 2 or x_fp4.stride(1) != 1:
        raise ValueError("x_fp4 must be uint8 [M, K/2] with unit stride along K")
    M, K = x_fp4.shape[0], x_fp4.shape[1] * 2
    if (x_scales.dtype != torch.uint8 or x_scales.dim() != 2 or x_scales.shape != (M, K // 32)
            or x_scales.stride(1) != 1):
        raise ValueError("x_scales must be uint8 [M, K/32] with unit stride along the blocks")
    dev = x_fp4.device
    if x_scales.device != dev:
        raise ValueError("x_scales must be on the device of x_fp4")
    _require_weight(w_pre, ws_pre, N, K, dev)
    _require_bias(bias, N, dev)
    code = {torch.bfloat16: MXFP4_OUT_BF16, torch.float32: MXFP4_OUT_F32}[out_dtype]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    else:
        _require_out(out, (M, N), out_dtype, dev)
    need = linear_prequantized_workspace_bytes(M, N, K)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace is not None:
        _require_bytes(workspace, "workspace", need, dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check("mxfp4_linear_prequantized", lib().mxfp4_linear_prequantized(
        _ptr(x_fp4), x_fp4.stride(0), _ptr(x_scales), x_scales.stride(0), _ptr(w_pre),
        _ptr(ws_pre), _ptr(bias), _ptr(out), out.stride(0), code, M, N, K, _ptr(workspace),
        ws_bytes, _stream(x_fp4.device)))
    return out


def a16wfp4_bmm(x: torch.Tensor, w_pre: torch.Tensor, ws_pre: torch.Tensor, N: int,
                out: Optional[torch.Tensor] = None, batch_major: bool = False,
                out_dtype: torch.dtype = torch.bfloat16):
    """x bf16 [B, M, K] (unit stride along K) x MXFP4 weights [B, N, K].

    Returns [B, M, N], or [M, B, N] when ``batch_major`` (a caller-supplied
    ``out`` may be any strided view with unit stride along N).
    """
    _require_cuda(x, "x")
    if x.dtype != torch.bfloat16 or x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("x must be a 3-D bf16 tensor with unit stride along K")
    B, M, K = x.shape
    _require_weight(w_pre, ws_pre, N, K, x.device, batch=B)
    code = {torch.bfloat16: MXFP4_OUT_BF16, torch.float32: MXFP4_OUT_F32}[out_dtype]
    shape = (M, B, N) if batch_major else (B, M, N)
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=x.device)
    else:
        _require_out(out, shape, out_dtype, x.device)
    if batch_major:
        sob, som = out.stride(1), out.stride(0)
    else:
        sob, som = out.stride(0), out.stride(1)
    _check("a16wfp4_bmm", lib().a16wfp4_bmm(
        _ptr(x), x.stride(0), x.stride(1), _ptr(w_pre), _ptr(ws_pre), _ptr(out), sob, som, code,
        B, M, N, K, _stream(x.device)))
    return out


@dataclass
class MXFP4Weight:
    """Preshuffled MXFP4 weight of ``batch`` matrices N x K (device tensors)."""
    w_pre: torch.Tensor
    ws_pre: torch.Tensor
    N: int
    K: int
    batch: int = 1


def quantize_weight(w: torch.Tensor) -> MXFP4Weight:
    """Load-time path: bf16 weight [N, K] or [B, N, K] -> MXFP4 in the GEMM layouts.

    One matrix (or N a multiple of 16) is quantised straight into the GEMM
    layout; otherwise row-major quantisation is followed by the preshuffle,
    which pads each batch entry to 16 rows.
    """
    _require_cuda(w, "w")
    w3 = w if w.dim() == 3 else w.unsqueeze(0)
    B, N, K = w3.shape
    flat = w3.reshape(B * N, K)
    if B == 1 or N % 16 == 0:
        w_pre, ws_pre = mxfp4_quant_1x32(flat, MXFP4_LAYOUT_GEMM)
    else:
        q, s = mxfp4_quant_1x32(flat, MXFP4_LAYOUT_ROWMAJOR)
        w_pre, ws_pre = mxfp4_preshuffle_weight(q, s, N, K, batch=B)
    return MXFP4Weight(w_pre, ws_pre, N, K, B)


def linear(x: torch.Tensor, weight: MXFP4Weight, bias: Optional[torch.Tensor] = None,
           out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """W4A4 linear: bf16 activations [..., K] quantised per 1x32, then the FP4 GEMM."""
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1])
    if x2.stride(1) != 1:
        x2 = x2.contiguous()
    y = mxfp4_linear(x2, weight.w_pre, weight.ws_pre, weight.N, bias, out_dtype)
    return y.reshape(*lead, weight.N)
