"""GPU parity of the GEMM with MXFP4 output (the next layer's activations
leave the GEMM quantised): the bytes equal the oracle's per-1x32
quantisation of the GEMM's own bf16 output (which the other GEMM tests hold
to the oracle's tolerance), and mxfp4_quant_1x32 (ROWMAJOR) of that output
on the GPU; for the small-M and the tiled kernel, with bias, ragged M and
row strides; and the result feeds mxfp4_linear_prequantized."""

import numpy as np
import pytest
import torch

import mxfp4_block_scaled_quant_amd as mx
from mxfp4_block_scaled_quant_amd import inputs
from oracle import quant as Q
from tests.helpers import dev_bf16, host_bf16_bits, host_u8, need_gpu

pytestmark = pytest.mark.gpu


def _run(M, N, K, path, seed=6, bias=True, pads=(0, 0), outliers=False):
    prob = inputs.linear_problem(M, N, K, seed, outliers=outliers, with_bias=bias)
    W = mx.quantize_weight(dev_bf16(prob["w"]))
    b = dev_bf16(prob["bias"]) if bias else None
    q, s = mx.mxfp4_quant_1x32(dev_bf16(prob["x"]), mx.MXFP4_LAYOUT_GEMM)
    oq = torch.zeros((M, N // 2 + pads[0]), dtype=torch.uint8, device="cuda")[:, :N // 2]
    os_ = torch.zeros((M, N // 32 + pads[1]), dtype=torch.uint8, device="cuda")[:, :N // 32]
    mx.set_gemm_path(path)
    try:
        mx.mxfp4_gemm_a4w4_mxfp4_out(q, s, W.w_pre, W.ws_pre, M, N, K, b, out_fp4=oq, out_scales=os_)
        y16 = mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.bfloat16)
    finally:
        mx.set_gemm_path(0)
    rq, rs = mx.mxfp4_quant_1x32(y16, mx.MXFP4_LAYOUT_ROWMAJOR)
    torch.cuda.synchronize()
    return prob, W, b, oq, os_, y16, rq, rs


CASES = [
    # name, M, N, K, path, kwargs
    ("smallM_16x1024x5120", 16, 1024, 5120, 1, dict(seed=0, outliers=True)),
    ("smallM_1x64x640", 1, 64, 640, 1, dict(pads=(4, 3))),
    ("smallM_37x96x4128", 37, 96, 4128, 1, dict(seed=5, pads=(8, 1))),
    ("smallM_64x320x1056", 64, 320, 1056, 1, dict(bias=False)),
    # the small-M kernel's persistent form, in steps of two strips
    ("persist_16x1024x5120", 16, 1024, 5120, 7, dict(seed=0, outliers=True)),
    ("persist_1x64x640", 1, 64, 640, 7, dict(pads=(4, 3))),
    ("persist_37x96x4128", 37, 96, 4128, 7, dict(seed=5, pads=(8, 1))),
    ("persist_64x320x1056", 64, 320, 1056, 7, dict(bias=False)),
    ("persist_20x8224x6144", 20, 8224, 6144, 7, dict(seed=3)),
    # up to 256 rows on few columns: the small-M kernel once per 64 rows
    ("rows_100x512x1056", 100, 512, 1056, 0, dict(outliers=True, pads=(4, 5))),
    ("rows_65x96x2080", 65, 96, 2080, 1, dict(seed=10)),
    ("tiled_300x512x1056", 300, 512, 1056, 2, dict(outliers=True, pads=(4, 5))),
    ("tiled256_300x512x1056", 300, 512, 1056, 3, dict(outliers=True, pads=(4, 5))),
    ("tiled_257x96x2080", 257, 96, 2080, 2, dict(seed=10)),
    ("tiled_37x288x4128", 37, 288, 4128, 2, dict(seed=5, bias=False)),
    # 128-wide output tiles (5), and with the split schedule forced (6)
    ("tiled128_300x512x1056", 300, 512, 1056, 5, dict(outliers=True, pads=(4, 5))),
    ("tiled128_split_257x96x2080", 257, 96, 2080, 6, dict(seed=10)),
    ("tiled128_37x288x4128", 37, 288, 4128, 5, dict(seed=5, bias=False)),
]


@pytest.mark.parametrize("name,M,N,K,path,kw", CASES, ids=[c[0] for c in CASES])
def test_mxfp4_out_is_the_quantised_bf16_output(name, M, N, K, path, kw):
    need_gpu()
    prob, W, b, oq, os_, y16, rq, rs = _run(M, N, K, path, **kw)
    q_ref, s_ref = Q.quant_1x32(host_bf16_bits(y16))              # the oracle's bytes
    assert np.array_equal(host_u8(oq), q_ref)
    assert np.array_equal(host_u8(os_), s_ref)
    assert np.array_equal(host_u8(oq), host_u8(rq))
    assert np.array_equal(host_u8(os_), host_u8(rs).reshape(M, N // 32))


@pytest.mark.parametrize("M,N,K", [(16, 14336, 5120), (2048, 5120, 14336)])
def test_mxfp4_out_full_size(M, N, K):
    # A decode and a prefill shape of the sweep: every byte against the GPU
    # quantisation of the bf16 output, sampled rows against the oracle.
    need_gpu()
    path = 1 if M <= 64 else 2
    prob, W, b, oq, os_, y16, rq, rs = _run(M, N, K, path, seed=3, bias=False, outliers=True)
    assert torch.equal(oq, rq)
    assert torch.equal(os_, rs.reshape(M, N // 32))
    rows = np.unique(np.r_[0, M - 1, np.random.default_rng(M).choice(M, 8)])
    q_ref, s_ref = Q.quant_1x32(host_bf16_bits(y16)[rows])
    assert np.array_equal(host_u8(oq)[rows], q_ref)
    assert np.array_equal(host_u8(os_)[rows], s_ref)


def test_mxfp4_out_feeds_the_next_layer():
    # layer 1 writes MXFP4, layer 2 reads it as a prequantised input: the
    # same as quantising layer 1's bf16 output and running layer 2.
    need_gpu()
    M, N1, N2, K = 16, 512, 256, 1056
    prob, W, b, oq, os_, y16, rq, rs = _run(M, N1, K, 1, outliers=True)
    W2 = mx.quantize_weight(dev_bf16(inputs.weights(N2, N1, 8)))
    z = mx.mxfp4_linear_prequantized(oq, os_, W2.w_pre, W2.ws_pre, N2, None, torch.float32)
    zr = mx.mxfp4_linear(y16, W2.w_pre, W2.ws_pre, N2, None, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(z.view(torch.int32), zr.view(torch.int32))
