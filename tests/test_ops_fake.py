"""The torch custom ops' fake implementations (no GPU): output shapes and
dtypes agree with the library's size queries, and tracing with symbolic
sizes goes through them."""

import pytest
import torch
from torch._subclasses.fake_tensor import FakeTensorMode
from torch.fx.experimental.proxy_tensor import make_fx

import mxfp4_block_scaled_quant_amd as mx
from mxfp4_block_scaled_quant_amd import ops  # noqa: F401  (registers torch.ops.mxfp4)

SHAPES = [(1, 32), (5, 96), (16, 5120), (17, 4128), (37, 4128), (300, 256), (8192, 14336)]


@pytest.mark.parametrize("M,K", SHAPES)
def test_quant_fake_shapes_match_size_queries(M, K):
    with FakeTensorMode():
        x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
        q, s = torch.ops.mxfp4.quant_1x32(x, mx.MXFP4_LAYOUT_GEMM)
        qr, sr = torch.ops.mxfp4.quant_1x32(x, mx.MXFP4_LAYOUT_ROWMAJOR)
    assert q.dtype == s.dtype == torch.uint8 and q.device.type == "cuda"
    assert q.numel() == mx.data_bytes(M, K, mx.MXFP4_LAYOUT_GEMM)
    assert s.numel() == mx.scale_bytes(M, K, mx.MXFP4_LAYOUT_GEMM)
    assert tuple(qr.shape) == (M, K // 2)
    assert sr.numel() == mx.scale_bytes(M, K, mx.MXFP4_LAYOUT_ROWMAJOR)


@pytest.mark.parametrize("B,N,K", [(1, 96, 4128), (1, 34816, 5120), (16, 512, 192), (16, 256, 512)])
def test_preshuffle_fake_shapes_match_size_queries(B, N, K):
    with FakeTensorMode():
        w = torch.empty((B * N * K // 2,), dtype=torch.uint8, device="cuda")
        s = torch.empty((B * N * K // 32,), dtype=torch.uint8, device="cuda")
        wp, sp = torch.ops.mxfp4.preshuffle_weight(w, s, N, K, B)
    assert wp.numel() == mx.weight_bytes(B, N, K)
    assert sp.numel() == mx.weight_scale_bytes(B, N, K)


def test_gemm_linear_bmm_fake_shapes():
    with FakeTensorMode():
        x = torch.empty((37, 4128), dtype=torch.bfloat16, device="cuda")
        w = torch.empty((mx.weight_bytes(1, 96, 4128),), dtype=torch.uint8, device="cuda")
        ws = torch.empty((mx.weight_scale_bytes(1, 96, 4128),), dtype=torch.uint8, device="cuda")
        q, s = torch.ops.mxfp4.quant_1x32(x, mx.MXFP4_LAYOUT_GEMM)
        y = torch.ops.mxfp4.gemm_a4w4(q, s, w, ws, 37, 96, 4128, None, torch.float32)
        z = torch.ops.mxfp4.linear(x, w, ws, 96)
        xb = torch.empty((16, 7, 512), dtype=torch.bfloat16, device="cuda")
        o1 = torch.ops.mxfp4.a16wfp4_bmm(xb, w, ws, 256, False)
        o2 = torch.ops.mxfp4.a16wfp4_bmm(xb, w, ws, 256, True)
    assert tuple(y.shape) == (37, 96) and y.dtype == torch.float32
    assert tuple(z.shape) == (37, 96) and z.dtype == torch.bfloat16
    assert tuple(o1.shape) == (16, 7, 256) and tuple(o2.shape) == (7, 16, 256)


def test_symbolic_trace_of_the_linear():
    # Quant + GEMM traced with a symbolic row count: the graph holds the two
    # ops and the output's size is the symbol.
    def f(x, w, ws):
        q, s = torch.ops.mxfp4.quant_1x32(x, mx.MXFP4_LAYOUT_GEMM)
        return torch.ops.mxfp4.gemm_a4w4(q, s, w, ws, x.shape[0], 96, x.shape[1], None, torch.bfloat16)

    x = torch.empty((37, 4128), dtype=torch.bfloat16, device="meta")
    w = torch.empty((mx.weight_bytes(1, 96, 4128),), dtype=torch.uint8, device="meta")
    ws = torch.empty((mx.weight_scale_bytes(1, 96, 4128),), dtype=torch.uint8, device="meta")
    g = make_fx(f, tracing_mode="symbolic")(x, w, ws)
    targets = [n.target for n in g.graph.nodes if n.op == "call_function"]
    assert torch.ops.mxfp4.quant_1x32.default in targets
    assert torch.ops.mxfp4.gemm_a4w4.default in targets
    out = [n for n in g.graph.nodes if n.op == "output"][0].args[0]
    val = out[0].meta["val"] if isinstance(out, (list, tuple)) else out.meta["val"]
    assert isinstance(val.shape[0], torch.SymInt) and val.shape[1] == 96
