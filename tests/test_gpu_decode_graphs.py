"""The small-M kernel's launch forms captured in a HIP graph: each replay,
with new inputs copied in and eager work (other calls, other inputs) in
between, is bitwise the eager call on the same inputs.

Forms: the persistent GEMM after the quantisation launch (mxfp4_linear,
M = 20), the persistent form encoding bf16 rows itself (mxfp4_linear, M = 3),
the persistent form gathering row-major operands (mxfp4_linear_prequantized,
M = 40), all at N = 24576, K = 5120 (six strips per compute unit); and one
strip per workgroup with four groups per round (N = 1000, K = 8704, M = 5)."""

import pytest
import torch

import mxfp4_block_scaled_quant_amd as mx
from mxfp4_block_scaled_quant_amd import inputs
from tests.helpers import dev_bf16, need_gpu

pytestmark = pytest.mark.gpu

_W = {}


def _weight(N, K):
    if (N, K) not in _W:
        _W[(N, K)] = (mx.quantize_weight(dev_bf16(inputs.weights(N, K, 31))), dev_bf16(inputs.bias(N, 31)))
    return _W[(N, K)]


def _prequant(x):
    M, K = x.shape
    q, s = mx.mxfp4_quant_1x32(x, mx.MXFP4_LAYOUT_ROWMAJOR)
    return q, s.view(M, K // 32)


CASES = [
    # name, M, N, K, prequantised input
    ("persist_linear_m20", 20, 24576, 5120, False),
    ("persist_fused_m3", 3, 24576, 5120, False),
    ("persist_rowmajor_m32", 32, 24576, 5120, True),
    ("permuted_rowmajor_m48", 48, 24576, 5120, True),   # permuted into the GEMM layouts first
    ("one_round_m5", 5, 1000, 8704, False),
]


@pytest.mark.parametrize("name,M,N,K,pre", CASES, ids=[c[0] for c in CASES])
def test_decode_graph_replays(name, M, N, K, pre):
    need_gpu()
    W, b = _weight(N, K)
    xs = [dev_bf16(inputs.activations(M, K, s, outliers=True)) for s in (1, 2, 3)]
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    if pre:
        ops = [_prequant(x) for x in xs]
        q_in, s_in = torch.empty_like(ops[0][0]), torch.empty_like(ops[0][1])
        call = lambda: mx.mxfp4_linear_prequantized(q_in, s_in, W.w_pre, W.ws_pre, N, b, torch.float32, out=out)
        eager = [mx.mxfp4_linear_prequantized(q, s, W.w_pre, W.ws_pre, N, b, torch.float32) for q, s in ops]

        def load(i):
            q_in.copy_(ops[i][0])
            s_in.copy_(ops[i][1])
    else:
        x_in = torch.empty_like(xs[0])
        ws = torch.empty(max(1, mx.linear_workspace_bytes(M, N, K)), dtype=torch.uint8, device="cuda")
        call = lambda: mx.mxfp4_linear(x_in, W.w_pre, W.ws_pre, N, b, torch.float32, out=out, workspace=ws)
        eager = [mx.mxfp4_linear(x, W.w_pre, W.ws_pre, N, b, torch.float32) for x in xs]

        def load(i):
            x_in.copy_(xs[i])
    load(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(6):
        i = rep % 3
        load(i)
        out.fill_(-1.0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager[i].view(torch.int32)), rep
        # eager work between replays: the same kind of call on other inputs
        e = mx.mxfp4_linear(xs[2 - i], W.w_pre, W.ws_pre, N, None, torch.bfloat16)
        torch.cuda.synchronize()
        del e
    del graph
