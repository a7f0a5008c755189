"""torch custom operators over the C ABI, with fake (meta) implementations.

The registered quantisation and GEMM ops of P2 §2 let the serving framework
trace, compile and capture the FP4 linear; these are their counterparts for
this library.  Each op's real implementation is the ctypes binding (every
step runs in the HIP kernels); its fake implementation only states output
shapes and dtypes, computed from the same layout rules as the library's size
queries, and works with symbolic sizes.

    torch.ops.mxfp4.quant_1x32(x, layout) -> (q, scales)
    torch.ops.mxfp4.preshuffle_weight(w_fp4, w_scales, N, K, batch) -> (w_pre, ws_pre)
    torch.ops.mxfp4.gemm_a4w4(a, a_scales, w_pre, ws_pre, M, N, K, bias, out_dtype) -> [M, N]
    torch.ops.mxfp4.linear(x, w_pre, ws_pre, N, bias, out_dtype) -> [M, N]
    torch.ops.mxfp4.gemm_a4w4_mxfp4_out(a, a_scales, w_pre, ws_pre, M, N, K, bias)
        -> (q [M, N/2], scales [M, N/32])
    torch.ops.mxfp4.shuffle_scales(scales, rows, K) -> GEMM-layout scales
    torch.ops.mxfp4.linear_prequantized(x_fp4, x_scales, w_pre, ws_pre, N, bias,
        out_dtype) -> [M, N]
    torch.ops.mxfp4.a16wfp4_bmm(x, w_pre, ws_pre, N, batch_major, out_dtype)
        -> [B, M, N] or [M, B, N]

None of the ops mutates its inputs or has an autograd formula (the path is
inference only).
"""

from __future__ import annotations

from typing import Optional, Tuple

import torch
from torch import Tensor

from . import (MXFP4_LAYOUT_GEMM, MXFP4_LAYOUT_ROWMAJOR, a16wfp4_bmm, mxfp4_gemm_a4w4,
               mxfp4_gemm_a4w4_mxfp4_out, mxfp4_linear, mxfp4_linear_prequantized, mxfp4_preshuffle_weight,
               mxfp4_quant_1x32, mxfp4_shuffle_scales)

__all__ = ["gemm_data_bytes", "gemm_scale_bytes"]


def _cdiv(a, b):
    return (a + b - 1) // b


def gemm_data_bytes(rows, K):
    """Bytes of packed FP4 in the GEMM data layout: whole 1 KiB units of
    16 rows x 128 K (rows and K padded)."""
    return _cdiv(rows, 16) * _cdiv(K, 128) * 1024


def gemm_scale_bytes(rows, K):
    """Bytes of E8M0 scales in the GEMM scale layout: 256-byte units of
    16 rows x 4 K-steps."""
    return _cdiv(rows, 16) * _cdiv(_cdiv(K, 128), 4) * 256


@torch.library.custom_op("mxfp4::quant_1x32", mutates_args=())
def quant_1x32(x: Tensor, layout: int) -> Tuple[Tensor, Tensor]:
    q, s = mxfp4_quant_1x32(x, layout)
    return q, s


@quant_1x32.register_fake
def _(x, layout):
    M, K = x.shape
    if layout == MXFP4_LAYOUT_ROWMAJOR:
        return (x.new_empty((M, K // 2), dtype=torch.uint8),
                x.new_empty((M * (K // 32),), dtype=torch.uint8))
    if layout == MXFP4_LAYOUT_GEMM:
        return (x.new_empty((gemm_data_bytes(M, K),), dtype=torch.uint8),
                x.new_empty((gemm_scale_bytes(M, K),), dtype=torch.uint8))
    raise ValueError(f"unknown layout {layout}")


@torch.library.custom_op("mxfp4::preshuffle_weight", mutates_args=())
def preshuffle_weight(w_fp4: Tensor, w_scales: Tensor, N: int, K: int,
                      batch: int = 1) -> Tuple[Tensor, Tensor]:
    w_pre, ws_pre = mxfp4_preshuffle_weight(w_fp4, w_scales, N, K, batch=batch)
    return w_pre, ws_pre


@preshuffle_weight.register_fake
def _(w_fp4, w_scales, N, K, batch=1):
    return (w_fp4.new_empty((batch * gemm_data_bytes(N, K),), dtype=torch.uint8),
            w_fp4.new_empty((batch * gemm_scale_bytes(N, K),), dtype=torch.uint8))


@torch.library.custom_op("mxfp4::gemm_a4w4", mutates_args=())
def gemm_a4w4(a: Tensor, a_scales: Tensor, w_pre: Tensor, ws_pre: Tensor, M: int, N: int,
              K: int, bias: Optional[Tensor] = None,
              out_dtype: torch.dtype = torch.bfloat16) -> Tensor:
    return mxfp4_gemm_a4w4(a, a_scales, w_pre, ws_pre, M, N, K, bias, out_dtype)


@gemm_a4w4.register_fake
def _(a, a_scales, w_pre, ws_pre, M, N, K, bias=None, out_dtype=torch.bfloat16):
    return a.new_empty((M, N), dtype=out_dtype)


@torch.library.custom_op("mxfp4::linear", mutates_args=())
def linear(x: Tensor, w_pre: Tensor, ws_pre: Tensor, N: int, bias: Optional[Tensor] = None,
           out_dtype: torch.dtype = torch.bfloat16) -> Tensor:
    return mxfp4_linear(x, w_pre, ws_pre, N, bias, out_dtype)


@linear.register_fake
def _(x, w_pre, ws_pre, N, bias=None, out_dtype=torch.bfloat16):
    return x.new_empty((x.shape[0], N), dtype=out_dtype)


@torch.library.custom_op("mxfp4::gemm_a4w4_mxfp4_out", mutates_args=())
def gemm_a4w4_mxfp4_out(a: Tensor, a_scales: Tensor, w_pre: Tensor, ws_pre: Tensor, M: int,
                        N: int, K: int, bias: Optional[Tensor] = None) -> Tuple[Tensor, Tensor]:
    q, s = mxfp4_gemm_a4w4_mxfp4_out(a, a_scales, w_pre, ws_pre, M, N, K, bias)
    return q, s


@gemm_a4w4_mxfp4_out.register_fake
def _(a, a_scales, w_pre, ws_pre, M, N, K, bias=None):
    return (a.new_empty((M, N // 2), dtype=torch.uint8), a.new_empty((M, N // 32), dtype=torch.uint8))


@torch.library.custom_op("mxfp4::shuffle_scales", mutates_args=())
def shuffle_scales(scales: Tensor, rows: int, K: int) -> Tensor:
    return mxfp4_shuffle_scales(scales, rows, K)


@shuffle_scales.register_fake
def _(scales, rows, K):
    return scales.new_empty((gemm_scale_bytes(rows, K),), dtype=torch.uint8)


@torch.library.custom_op("mxfp4::linear_prequantized", mutates_args=())
def linear_prequantized(x_fp4: Tensor, x_scales: Tensor, w_pre: Tensor, ws_pre: Tensor, N: int,
                        bias: Optional[Tensor] = None,
                        out_dtype: torch.dtype = torch.bfloat16) -> Tensor:
    return mxfp4_linear_prequantized(x_fp4, x_scales, w_pre, ws_pre, N, bias, out_dtype)


@linear_prequantized.register_fake
def _(x_fp4, x_scales, w_pre, ws_pre, N, bias=None, out_dtype=torch.bfloat16):
    return x_fp4.new_empty((x_fp4.shape[0], N), dtype=out_dtype)


@torch.library.custom_op("mxfp4::a16wfp4_bmm", mutates_args=())
def bmm(x: Tensor, w_pre: Tensor, ws_pre: Tensor, N: int, batch_major: bool = False,
        out_dtype: torch.dtype = torch.bfloat16) -> Tensor:
    return a16wfp4_bmm(x, w_pre, ws_pre, N, batch_major=batch_major, out_dtype=out_dtype)


@bmm.register_fake
def _(x, w_pre, ws_pre, N, batch_major=False, out_dtype=torch.bfloat16):
    B, M, _ = x.shape
    shape = (M, B, N) if batch_major else (B, M, N)
    return x.new_empty(shape, dtype=out_dtype)
