"""The Python binding checks every caller-supplied tensor on the host before
any launch: operand sizes against the library's size queries, output shape,
dtype, device and unit stride, bias shape and dtype, workspace size.  Run on
the CPU with meta tensors (no data, no launch): each bad argument must raise
ValueError before the library is asked to do any work."""

import pytest
import torch

import mxfp4_block_scaled_quant_amd as mx

META = torch.device("meta")


@pytest.fixture(autouse=True)
def _meta_is_a_device(monkeypatch):
    # meta tensors stand in for device tensors here: only the checks run
    monkeypatch.setattr(mx, "_require_cuda", lambda t, name: None)


def u8(n):
    return torch.empty(n, dtype=torch.uint8, device=META)


def operands(M, N, K):
    return (u8(mx.data_bytes(M, K, mx.MXFP4_LAYOUT_GEMM)), u8(mx.scale_bytes(M, K, mx.MXFP4_LAYOUT_GEMM)),
            u8(mx.weight_bytes(1, N, K)), u8(mx.weight_scale_bytes(1, N, K)))


def _raises(fn, *a, **kw):
    with pytest.raises(ValueError):
        fn(*a, **kw)


def test_gemm_rejects_bad_operands_and_outputs():
    M, N, K = 16, 1024, 5120
    a, s, w, ws = operands(M, N, K)
    _raises(mx.mxfp4_gemm_a4w4, a[:-1], s, w, ws, M, N, K)              # activations short
    _raises(mx.mxfp4_gemm_a4w4, a, s[:-1], w, ws, M, N, K)
    _raises(mx.mxfp4_gemm_a4w4, a, s, w[:-16], ws, M, N, K)            # weight short
    _raises(mx.mxfp4_gemm_a4w4, a, s, w, ws[:-4], M, N, K)
    _raises(mx.mxfp4_gemm_a4w4, a.view(torch.int8), s, w, ws, M, N, K)  # not uint8
    bad_bias = torch.empty(N - 1, dtype=torch.bfloat16, device=META)
    _raises(mx.mxfp4_gemm_a4w4, a, s, w, ws, M, N, K, bad_bias)
    f32_bias = torch.empty(N, dtype=torch.float32, device=META)
    _raises(mx.mxfp4_gemm_a4w4, a, s, w, ws, M, N, K, f32_bias)
    # a bf16 out passed with out_dtype=float32 would be written past its end
    out16 = torch.empty((M, N), dtype=torch.bfloat16, device=META)
    _raises(mx.mxfp4_gemm_a4w4, a, s, w, ws, M, N, K, None, torch.float32, out=out16)
    _raises(mx.mxfp4_gemm_a4w4, a, s, w, ws, M, N, K, None, torch.bfloat16,
            out=torch.empty((M - 1, N), dtype=torch.bfloat16, device=META))
    strided = torch.empty((M, 2 * N), dtype=torch.bfloat16, device=META)[:, ::2]
    _raises(mx.mxfp4_gemm_a4w4, a, s, w, ws, M, N, K, None, torch.bfloat16, out=strided)
    # a workspace smaller than the split schedule asks
    Mp, Np, Kp = 8192, 5120, 14336
    need = mx.gemm_workspace_bytes(Mp, Np, Kp)
    assert need > 0
    ap, sp, wp, wsp = operands(Mp, Np, Kp)
    _raises(mx.mxfp4_gemm_a4w4, ap, sp, wp, wsp, Mp, Np, Kp, workspace=u8(need - 1))


def test_linear_and_prequantized_reject_bad_arguments():
    M, N, K = 17, 1024, 5120
    x = torch.empty((M, K), dtype=torch.bfloat16, device=META)
    _, _, w, ws = operands(M, N, K)
    _raises(mx.mxfp4_linear, x, w[:-1], ws, N)
    _raises(mx.mxfp4_linear, x, w, ws, N, out=torch.empty((M, N), dtype=torch.float32, device=META))
    _raises(mx.mxfp4_linear, x, w, ws, N, workspace=u8(mx.linear_workspace_bytes(M, N, K) - 1))
    _raises(mx.mxfp4_linear, x.to(torch.float32), w, ws, N)
    xq = torch.empty((M, K // 2), dtype=torch.uint8, device=META)
    xs = torch.empty((M, K // 32), dtype=torch.uint8, device=META)
    _raises(mx.mxfp4_linear_prequantized, xq, xs, w, ws[:-4], N)
    _raises(mx.mxfp4_linear_prequantized, xq, xs, w, ws, N,
            out=torch.empty((M, N + 1), dtype=torch.bfloat16, device=META))


def test_mxfp4_out_and_quant_reject_bad_outputs():
    M, N, K = 16, 1024, 5120
    a, s, w, ws = operands(M, N, K)
    _raises(mx.mxfp4_gemm_a4w4_mxfp4_out, a, s, w, ws, M, N, K,
            out_fp4=torch.empty((M, N // 2 - 1), dtype=torch.uint8, device=META))
    _raises(mx.mxfp4_gemm_a4w4_mxfp4_out, a, s, w, ws, M, N, K,
            out_scales=torch.empty((M, N // 32), dtype=torch.int8, device=META))
    x = torch.empty((M, K), dtype=torch.bfloat16, device=META)
    _raises(mx.mxfp4_quant_1x32, x, mx.MXFP4_LAYOUT_GEMM, q=u8(mx.data_bytes(M, K, 1) - 1))
    _raises(mx.mxfp4_quant_1x32, x, mx.MXFP4_LAYOUT_GEMM, scales=u8(mx.scale_bytes(M, K, 1) - 1))
    _raises(mx.mxfp4_quant_1x32, x, mx.MXFP4_LAYOUT_ROWMAJOR,
            q=torch.empty((M, K // 2 - 2), dtype=torch.uint8, device=META))
    _raises(mx.mxfp4_shuffle_scales, torch.empty((M, K // 32), dtype=torch.uint8, device=META), M, K,
            out=u8(mx.scale_bytes(M, K, 1) - 1))


def test_bmm_rejects_bad_weights_and_outputs():
    B, M, N, K = 16, 64, 256, 512
    x = torch.empty((B, M, K), dtype=torch.bfloat16, device=META)
    w, ws = u8(mx.weight_bytes(B, N, K)), u8(mx.weight_scale_bytes(B, N, K))
    _raises(mx.a16wfp4_bmm, x, w[:-1], ws, N)
    _raises(mx.a16wfp4_bmm, x, u8(mx.weight_bytes(1, N, K)), u8(mx.weight_scale_bytes(1, N, K)), N)
    # [B, M, N] output passed for the batch-major form, and the reverse
    _raises(mx.a16wfp4_bmm, x, w, ws, N, out=torch.empty((B, M, N), dtype=torch.bfloat16, device=META),
            batch_major=True)
    _raises(mx.a16wfp4_bmm, x, w, ws, N, out=torch.empty((M, B, N), dtype=torch.bfloat16, device=META))
    _raises(mx.a16wfp4_bmm, x, w, ws, N, out=torch.empty((B, M, N), dtype=torch.float32, device=META))
