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
  the quantisation fused into the GEMM kernel for M <= 16
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
    "mxfp4_gemm_a4w4_mxfp4_out": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_vp,
                                           _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_size, _c_vp]),
    "mxfp4_shuffle_scales": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp]),
    "mxfp4_linear_prequantized_workspace_bytes": (_c_size, [_c_i64, _c_i64, _c_i64]),
    "mxfp4_linear_prequantized": (_c_int, [_c_vp, _c_i64, _c_vp, _c_i64, _c_vp, _c_vp, _c_vp,
                                           _c_vp, _c_i64, _c_int, _c_i64, _c_i64, _c_i64,
                                           _c_vp, _c_size, _c_vp]),
    "a16wfp4_bmm": (_c_int, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_int,
                             _c_i64, _c_i64, _c_i64, _c_i64, _c_vp]),
    "mxfp4_debug_set_gemm_path": (_c_int, [_c_int]),
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


def data_bytes(rows: int, K: int, layout: int) -> int:
    return int(lib().mxfp4_data_bytes(rows, K, layout))


def scale_bytes(rows: int, K: int, layout: int) -> int:
    return int(lib().mxfp4_scale_bytes(rows, K, layout))


def weight_bytes(batch: int, N: int, K: int) -> int:
    return int(lib().mxfp4_weight_bytes(batch, N, K))


def weight_scale_bytes(batch: int, N: int, K: int) -> int:
    return int(lib().mxfp4_weight_scale_bytes(batch, N, K))


def set_gemm_path(path: int) -> None:
    """Test hook: 1 forces the small-M kernel (M <= 64), 2 the tiled kernel, 0 = by M;
    3 the tiled kernel on whole 256-wide tiles only, 4 with the split (split-K)
    schedule; 5 and 6 the same with 128-wide tiles."""
    _check("mxfp4_debug_set_gemm_path", lib().mxfp4_debug_set_gemm_path(path))


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
    if scales is None:
        scales = torch.empty(scale_bytes(M, K, layout), dtype=torch.uint8, device=x.device)
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


def mxfp4_gemm_a4w4(a_fp4: torch.Tensor, a_scales: torch.Tensor, w_pre: torch.Tensor,
                    ws_pre: torch.Tensor, M: int, N: int, K: int,
                    bias: Optional[torch.Tensor] = None,
                    out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None):
    """out[M, N] = dq(A) dq(W)^T (+ bias), bf16 or fp32; A and W in the GEMM layouts."""
    _require_cuda(a_fp4, "a_fp4")
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() != N):
        raise ValueError("bias must be bf16 [N]")
    code = {torch.bfloat16: MXFP4_OUT_BF16, torch.float32: MXFP4_OUT_F32}[out_dtype]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_fp4.device)
    ws_bytes = int(lib().mxfp4_gemm_workspace_bytes(M, N, K))
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=a_fp4.device) if ws_bytes else None
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
    allocated here when needed and not given; M <= 16 needs none.
    """
    _require_cuda(x, "x")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit stride along K")
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() != N):
        raise ValueError("bias must be bf16 [N]")
    M, K = x.shape
    code = {torch.bfloat16: MXFP4_OUT_BF16, torch.float32: MXFP4_OUT_F32}[out_dtype]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    need = linear_workspace_bytes(M, N, K)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check("mxfp4_linear", lib().mxfp4_linear(
        _ptr(x), x.stride(0), _ptr(w_pre), _ptr(ws_pre), _ptr(bias), _ptr(out), out.stride(0),
        code, M, N, K, _ptr(workspace), ws_bytes, _stream(x.device)))
    return out


def mxfp4_gemm_a4w4_mxfp4_out(a_fp4: torch.Tensor, a_scales: torch.Tensor, w_pre: torch.Tensor,
                              ws_pre: torch.Tensor, M: int, N: int, K: int,
                              bias: Optional[torch.Tensor] = None,
                              out_fp4: Optional[torch.Tensor] = None,
                              out_scales: Optional[torch.Tensor] = None):
    """(q [M, N/2], scales [M, N/32]) uint8: the GEMM's rows quantised per 1x32
    along N (bitwise mxfp4_quant_1x32 of the bf16 output, ROWMAJOR)."""
    _require_cuda(a_fp4, "a_fp4")
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() != N):
        raise ValueError("bias must be bf16 [N]")
    if out_fp4 is None:
        out_fp4 = torch.empty((M, N // 2), dtype=torch.uint8, device=a_fp4.device)
    if out_scales is None:
        out_scales = torch.empty((M, N // 32), dtype=torch.uint8, device=a_fp4.device)
    for t, name in ((out_fp4, "out_fp4"), (out_scales, "out_scales")):
        if t.dtype != torch.uint8 or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} must be 2-D uint8 with unit stride along N")
    ws_bytes = int(lib().mxfp4_gemm_workspace_bytes(M, N, K))
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=a_fp4.device) if ws_bytes else None
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
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() != N):
        raise ValueError("bias must be bf16 [N]")
    code = {torch.bfloat16: MXFP4_OUT_BF16, torch.float32: MXFP4_OUT_F32}[out_dtype]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x_fp4.device)
    need = linear_prequantized_workspace_bytes(M, N, K)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x_fp4.device)
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
    code = {torch.bfloat16: MXFP4_OUT_BF16, torch.float32: MXFP4_OUT_F32}[out_dtype]
    if out is None:
        if batch_major:
            out = torch.empty((M, B, N), dtype=out_dtype, device=x.device)
        else:
            out = torch.empty((B, M, N), dtype=out_dtype, device=x.device)
    if batch_major:
        sob, som = out.stride(1), out.stride(0)
    else:
        sob, som = out.stride(0), out.stride(1)
    if out.stride(-1) != 1:
        raise ValueError("out must have unit stride along N")
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
