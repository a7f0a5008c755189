"""The entry point that allocates nothing (mxfp4_linear_noalloc), called
through the C ABI: its output against mxfp4_linear's on the same operands,
on calls in a row through the library's shared scratch, each later call
with a smaller input than the one before it (so a stale byte of an earlier
call would show), bitwise where mxfp4_linear runs the same kernels (every
shape here: the small-M kernel, and whole tiles of the large-M kernel), and
within the oracle's bar.  Also: a shape whose quantised activations exceed
the scratch is refused before any launch."""

import numpy as np
import pytest
import torch

import mxfp4_block_scaled_quant_amd as mx
from mxfp4_block_scaled_quant_amd import inputs
from tests.helpers import dev_bf16, host_bf16_bits, need_gpu

pytestmark = pytest.mark.gpu


def _pair(prob, N, W, out_dtype):
    x = dev_bf16(prob["x"])
    b = None if prob["bias"] is None else dev_bf16(prob["bias"])
    a = mx.mxfp4_linear_noalloc(x, W.w_pre, W.ws_pre, N, b, out_dtype)
    r = mx.mxfp4_linear(x, W.w_pre, W.ws_pre, N, b, out_dtype)
    torch.cuda.synchronize()
    return a, r


def test_noalloc_matches_linear_on_calls_in_a_row():
    need_gpu()
    from tests.test_gpu_gemm import _check
    # (M, N, K, seed, edge): 300 rows (large-M kernel, whole tiles: what
    # mxfp4_linear also runs at this shape), then 37, then 16 (small-M
    # kernel through the scratch), then 3 (fused: no scratch)
    calls = [(300, 128, 256, 5, True), (37, 96, 4128, 5, True), (16, 1024, 5120, 0, False), (3, 96, 4128, 6, False)]
    assert mx.gemm_workspace_bytes(300, 128, 256) == 0      # no split schedule for the reference either
    for M, N, K, seed, edge in calls:
        prob = inputs.linear_problem(M, N, K, seed, edge=edge, outliers=not edge, with_bias=True)
        W = mx.quantize_weight(dev_bf16(prob["w"]))
        a32, r32 = _pair(prob, N, W, torch.float32)
        a16, r16 = _pair(prob, N, W, torch.bfloat16)
        assert np.array_equal(a32.cpu().numpy().view(np.uint32), r32.cpu().numpy().view(np.uint32)), M
        assert np.array_equal(host_bf16_bits(a16), host_bf16_bits(r16)), M
        _check(prob, a32.cpu().numpy(), host_bf16_bits(a16))


def test_noalloc_refuses_shapes_beyond_its_scratch():
    need_gpu()
    M, N, K = 4416, 128, 14336            # 276 strips of 112 KiB codes + 7 KiB scales: past 32 MiB
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    W = mx.quantize_weight(torch.zeros((N, K), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(mx.MXFP4Error) as e:
        mx.mxfp4_linear_noalloc(x, W.w_pre, W.ws_pre, N)
    assert e.value.status == 4
