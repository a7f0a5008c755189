"""GPU checks of the torch custom ops: torch.library.opcheck (schema, fake vs
real, dispatch), torch.compile through the fake implementations with
dynamic sizes, and capture in a CUDA (HIP) graph -- each bitwise equal to
the direct binding calls -- and the ops' own outputs held to the oracle."""

import numpy as np
import pytest
import torch

import mxfp4_block_scaled_quant_amd as mx
from mxfp4_block_scaled_quant_amd import inputs, ops  # noqa: F401
from tests.helpers import dev_bf16, need_gpu

pytestmark = pytest.mark.gpu


def _problem(M=37, N=96, K=4128):
    p = inputs.linear_problem(M, N, K, 5, edge=True, with_bias=True)
    W = mx.quantize_weight(dev_bf16(p["w"]))
    return dev_bf16(p["x"]), W, dev_bf16(p["bias"])


def test_opcheck_every_op():
    need_gpu()
    x, W, b = _problem()
    M, K = x.shape
    N = W.N
    q, s = mx.mxfp4_quant_1x32(x, mx.MXFP4_LAYOUT_GEMM)
    qr, sr = mx.mxfp4_quant_1x32(x, mx.MXFP4_LAYOUT_ROWMAJOR)
    xb = dev_bf16(inputs.bmm_problem(4, 9, 64, 192, 4)["x"])
    Wb = mx.quantize_weight(dev_bf16(inputs.bmm_problem(4, 9, 64, 192, 4)["w"]))
    cases = [
        (torch.ops.mxfp4.quant_1x32.default, (x, mx.MXFP4_LAYOUT_GEMM)),
        (torch.ops.mxfp4.quant_1x32.default, (x, mx.MXFP4_LAYOUT_ROWMAJOR)),
        (torch.ops.mxfp4.preshuffle_weight.default, (qr, sr, M, K, 1)),
        (torch.ops.mxfp4.gemm_a4w4.default, (q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.float32)),
        (torch.ops.mxfp4.linear.default, (x, W.w_pre, W.ws_pre, N, b, torch.bfloat16)),
        (torch.ops.mxfp4.linear.default, (x[:1], W.w_pre, W.ws_pre, N, None, torch.float32)),
        (torch.ops.mxfp4.a16wfp4_bmm.default, (xb, Wb.w_pre, Wb.ws_pre, 64, True, torch.bfloat16)),
        (torch.ops.mxfp4.shuffle_scales.default, (sr.reshape(M, K // 32), M, K)),
        (torch.ops.mxfp4.gemm_a4w4_mxfp4_out.default, (q, s, W.w_pre, W.ws_pre, M, 64, K, None)),
        (torch.ops.mxfp4.linear_prequantized.default,
         (qr, sr.reshape(M, K // 32), W.w_pre, W.ws_pre, N, b, torch.float32)),
        (torch.ops.mxfp4.linear_prequantized.default,
         (qr[:5], sr.reshape(M, K // 32)[:5], W.w_pre, W.ws_pre, N, None, torch.bfloat16)),
    ]
    for op, args in cases:
        torch.library.opcheck(op, args, test_utils=("test_schema", "test_faketensor",
                                                    "test_aot_dispatch_dynamic"))


def test_compile_dynamic_matches_eager():
    need_gpu()
    x, W, b = _problem()

    def f(x):
        q, s = torch.ops.mxfp4.quant_1x32(x, mx.MXFP4_LAYOUT_GEMM)
        y = torch.ops.mxfp4.gemm_a4w4(q, s, W.w_pre, W.ws_pre, x.shape[0], W.N, x.shape[1], b,
                                      torch.float32)
        z = torch.ops.mxfp4.linear(x, W.w_pre, W.ws_pre, W.N, b, torch.float32)
        return y, z

    fc = torch.compile(f, backend="aot_eager", dynamic=True, fullgraph=True)
    for M in (37, 3, 16, 1):
        y, z = fc(x[:M])
        ye, ze = f(x[:M])
        assert torch.equal(y.view(torch.int32), ye.view(torch.int32))
        assert torch.equal(z.view(torch.int32), ze.view(torch.int32))


def test_graph_capture_replays():
    # linear at M = 1 (the fused kernel) and M = 37 (quant into a workspace,
    # then the GEMM) captured once and replayed with eager work in between;
    # every replay equals the eager result.
    need_gpu()
    x, W, b = _problem()
    for M in (1, 37):
        xin = x[:M].clone()
        ref = torch.ops.mxfp4.linear(xin, W.w_pre, W.ws_pre, W.N, b, torch.float32)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            torch.ops.mxfp4.linear(xin, W.w_pre, W.ws_pre, W.N, b, torch.float32)   # warm
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            out = torch.ops.mxfp4.linear(xin, W.w_pre, W.ws_pre, W.N, b, torch.float32)
        for _ in range(3):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
            _ = torch.ops.mxfp4.linear(x, W.w_pre, W.ws_pre, W.N, None, torch.bfloat16)  # eager work
            torch.cuda.synchronize()


def test_ops_meet_the_oracle():
    # The ops' own outputs held to the oracle directly (not only through the
    # binding calls they equal): quantisation bytes exactly, the GEMM and the
    # linear within the GEMM bar, the BMM within its bar.
    need_gpu()
    from oracle import linalg as G
    from oracle import quant as Q
    from tests.helpers import check_f32_tolerance, host_u8
    from tests.test_gpu_gemm import _check

    M, N, K = 37, 96, 4128
    p = inputs.linear_problem(M, N, K, 5, edge=True, with_bias=True)
    x, b = dev_bf16(p["x"]), dev_bf16(p["bias"])
    W = mx.quantize_weight(dev_bf16(p["w"]))
    qr, sr = torch.ops.mxfp4.quant_1x32(x, mx.MXFP4_LAYOUT_ROWMAJOR)
    q_ref, s_ref = Q.quant_1x32(p["x"])
    assert np.array_equal(host_u8(qr), q_ref)
    assert np.array_equal(host_u8(sr).reshape(M, K // 32), s_ref)
    q, s = torch.ops.mxfp4.quant_1x32(x, mx.MXFP4_LAYOUT_GEMM)
    y32 = torch.ops.mxfp4.gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.float32)
    y16 = torch.ops.mxfp4.gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.bfloat16)
    torch.cuda.synchronize()
    _check(p, y32.cpu().numpy(), y16.cpu().view(torch.int16).numpy().view(np.uint16))
    for rows in (1, 16, M):
        pr = dict(p, x=p["x"][:rows])
        z32 = torch.ops.mxfp4.linear(x[:rows], W.w_pre, W.ws_pre, N, b, torch.float32)
        z16 = torch.ops.mxfp4.linear(x[:rows], W.w_pre, W.ws_pre, N, b, torch.bfloat16)
        torch.cuda.synchronize()
        _check(pr, z32.cpu().numpy(), z16.cpu().view(torch.int16).numpy().view(np.uint16))
    pb = inputs.bmm_problem(4, 9, 64, 192, 4)
    Wb = mx.quantize_weight(dev_bf16(pb["w"]))
    o = torch.ops.mxfp4.a16wfp4_bmm(dev_bf16(pb["x"]), Wb.w_pre, Wb.ws_pre, 64, True, torch.float32)
    torch.cuda.synchronize()
    qw, sw = Q.quant_1x32(pb["w"].reshape(4 * 64, 192))
    o_ref, S = G.bmm_a16wfp4(pb["x"], qw.reshape(4, 64, 96), sw.reshape(4, 64, 6))
    check_f32_tolerance(o.cpu().numpy().transpose(1, 0, 2), o_ref, S)
