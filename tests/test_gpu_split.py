"""GPU parity of the large-M kernel's split (split-K) schedule.

A tile split along K between workgroups meets in the workspace: the last
workgroup to finish a slice adds the others in K order.  Forced on small
shapes (every tile is cut into as many slices as idle workgroups allow, at
most one per group of 4 K-steps: 3, 5 and 9 slices per tile here), the
results, at both output-tile widths (256 and 128 columns), must meet the
oracle's bar like the whole-tile schedule's
(tests/test_gpu_gemm.py), be identical run to run (the sum does not depend
on which slice finishes last), not read a part left
by an earlier call, and replay correctly from a captured graph (the
workspace's counters are cleared by a kernel the graph holds).  The
automatic schedule at the sweep's shapes is covered by the full-size tests
there."""

import numpy as np
import pytest
import torch

import mxfp4_block_scaled_quant_amd as mx
from mxfp4_block_scaled_quant_amd import inputs
from oracle import quant as Q
from tests.helpers import dev_bf16, host_bf16_bits, host_u8, need_gpu
from tests.test_gpu_gemm import _check, _run, assert_no_giveup

pytestmark = pytest.mark.gpu

SPLIT, WHOLE = 4, 3   # set_gemm_path: tiled kernel, split schedule / whole tiles only
SPLIT128, WHOLE128 = 6, 5   # the same with 128-wide output tiles

CASES = [
    # name, M, N, K, problem kwargs: 2 x 3 tiles of 3 groups (3 slices each),
    # 2 x 2 of 5 (5 slices), one ragged tile of 9 (9 slices)
    ("parts3_300x520x1056", 300, 520, 1056, dict(seed=6, outliers=True, with_bias=True)),
    ("parts5_257x257x2080", 257, 257, 2080, dict(seed=10, outliers=True)),
    ("parts9_37x96x4128", 37, 96, 4128, dict(seed=5, edge=True, with_bias=True)),
]


@pytest.mark.parametrize("split,whole", [(SPLIT, WHOLE), (SPLIT128, WHOLE128)], ids=["w256", "w128"])
@pytest.mark.parametrize("name,M,N,K,kw", CASES, ids=[c[0] for c in CASES])
def test_split_matches_oracle(name, M, N, K, kw, split, whole):
    need_gpu()
    print(f"[split] {name} path {split}", flush=True)
    prob = inputs.linear_problem(M, N, K, **kw)
    y32, y16 = _run(prob, split)
    _check(prob, y32, y16)
    # the same operands on whole tiles: both within the oracle's bar, and
    # apart only by the order of the fp32 sums
    w32, w16 = _run(prob, whole)
    _check(prob, w32, w16)


@pytest.mark.parametrize("split", [SPLIT, SPLIT128], ids=["w256", "w128"])
def test_split_identical_run_to_run_and_no_stale_parts(split):
    # Two problems of one shape alternate through the same workspace sizes:
    # A, B, A.  Each result meets the oracle's bar, and the two runs of A are
    # bitwise equal (the parts are summed in K order, and nothing of B's
    # parts is read).
    need_gpu()
    M, N, K = 37, 96, 4128
    pa = inputs.linear_problem(M, N, K, 5, edge=True, with_bias=True)
    pb = inputs.linear_problem(M, N, K, 7, outliers=True, with_bias=True)
    a1 = _run(pa, split)
    b1 = _run(pb, split)
    a2 = _run(pa, split)
    _check(pa, *a1)
    _check(pb, *b1)
    assert np.array_equal(a1[0].view(np.uint32), a2[0].view(np.uint32))
    assert np.array_equal(a1[1], a2[1])
    assert not np.array_equal(a1[1], b1[1])


def test_split_mxfp4_out_is_the_quantised_bf16_output():
    # The MXFP4-output epilogue runs after the same combine: its bytes are
    # the per-1x32 quantisation of the bf16 output of the same schedule.
    need_gpu()
    M, N, K = 300, 512, 1056
    prob = inputs.linear_problem(M, N, K, 6, outliers=True, with_bias=True)
    W = mx.quantize_weight(dev_bf16(prob["w"]))
    b = dev_bf16(prob["bias"])
    q, s = mx.mxfp4_quant_1x32(dev_bf16(prob["x"]), mx.MXFP4_LAYOUT_GEMM)
    mx.set_gemm_path(SPLIT)
    try:
        need = mx.gemm_workspace_bytes(M, N, K)
        assert need > 0
        ws = [torch.empty(need, dtype=torch.uint8, device="cuda") for _ in range(2)]
        oq, os_ = mx.mxfp4_gemm_a4w4_mxfp4_out(q, s, W.w_pre, W.ws_pre, M, N, K, b, workspace=ws[0])
        y16 = mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.bfloat16, workspace=ws[1])
    finally:
        mx.set_gemm_path(0)
    torch.cuda.synchronize()
    assert_no_giveup(*ws)
    q_ref, s_ref = Q.quant_1x32(host_bf16_bits(y16))
    assert np.array_equal(host_u8(oq), q_ref)
    assert np.array_equal(host_u8(os_), s_ref)


@pytest.mark.parametrize("split", [SPLIT, SPLIT128], ids=["w256", "w128"])
def test_split_linear_entry_points(split):
    # mxfp4_linear (quantisation into the workspace, then the GEMM with its
    # part of the workspace after it) and mxfp4_linear_prequantized.
    need_gpu()
    M, N, K = 257, 257, 2080
    prob = inputs.linear_problem(M, N, K, 10, outliers=True, with_bias=True)
    W = mx.quantize_weight(dev_bf16(prob["w"]))
    b = dev_bf16(prob["bias"])
    x = dev_bf16(prob["x"])
    mx.set_gemm_path(split)
    try:
        assert mx.linear_workspace_bytes(M, N, K) > mx.linear_workspace_bytes(M, N, 256)
        y32 = mx.mxfp4_linear(x, W.w_pre, W.ws_pre, N, b, torch.float32)
        y16 = mx.mxfp4_linear(x, W.w_pre, W.ws_pre, N, b, torch.bfloat16)
        xq, xs = mx.mxfp4_quant_1x32(x, mx.MXFP4_LAYOUT_ROWMAJOR)
        p32 = mx.mxfp4_linear_prequantized(xq, xs.reshape(M, K // 32), W.w_pre, W.ws_pre, N, b, torch.float32)
    finally:
        mx.set_gemm_path(0)
    torch.cuda.synchronize()
    _check(prob, y32.cpu().numpy(), host_bf16_bits(y16))
    assert np.array_equal(y32.cpu().numpy().view(np.uint32), p32.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("split", [SPLIT, SPLIT128], ids=["w256", "w128"])
def test_split_graph_replays(split):
    # The counter-clearing kernel and the GEMM captured together; replays
    # with new operands copied in between (eager work and synchronisation
    # between replays), each checked against the eager call on the same
    # operands, bitwise.
    need_gpu()
    M, N, K = 300, 520, 1056
    probs = [inputs.linear_problem(M, N, K, s, outliers=True, with_bias=True) for s in (6, 8, 9)]
    W = mx.quantize_weight(dev_bf16(probs[0]["w"]))
    b = dev_bf16(probs[0]["bias"])
    qs = [mx.mxfp4_quant_1x32(dev_bf16(p["x"]), mx.MXFP4_LAYOUT_GEMM) for p in probs]
    q_in = torch.empty_like(qs[0][0])
    s_in = torch.empty_like(qs[0][1])
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    mx.set_gemm_path(split)
    try:
        gws = torch.empty(mx.gemm_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
        assert gws.numel() > 0
        eager = [mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.float32) for q, s in qs]
        q_in.copy_(qs[0][0])
        s_in.copy_(qs[0][1])
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            mx.mxfp4_gemm_a4w4(q_in, s_in, W.w_pre, W.ws_pre, M, N, K, b, torch.float32, out=out, workspace=gws)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            mx.mxfp4_gemm_a4w4(q_in, s_in, W.w_pre, W.ws_pre, M, N, K, b, torch.float32, out=out, workspace=gws)
        for rep in range(6):
            i = rep % 3
            q_in.copy_(qs[i][0])
            s_in.copy_(qs[i][1])
            out.fill_(-1.0)
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int32), eager[i].view(torch.int32)), rep
            assert_no_giveup(gws)
            # eager work between replays, through a workspace of its own
            e = mx.mxfp4_gemm_a4w4(qs[2 - i][0], qs[2 - i][1], W.w_pre, W.ws_pre, M, N, K, b, torch.float32)
            torch.cuda.synchronize()
            assert torch.equal(e.view(torch.int32), eager[2 - i].view(torch.int32)), rep
    finally:
        mx.set_gemm_path(0)
    # (every call used the first problem's weight and bias)
    ref = {"x": probs[1]["x"], "w": probs[0]["w"], "bias": probs[0]["bias"]}
    _check(ref, eager[1].cpu().numpy(), host_bf16_bits(eager[1].to(torch.bfloat16)))
    del graph
