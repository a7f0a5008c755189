"""GPU parity of the prequantised-input path: activations quantised by a
producer arrive as row-major packed FP4 + row-major E8M0 scales.

* mxfp4_shuffle_scales: bytewise the oracle's GEMM scale layout (0x7F
  padding), with and without a row stride.
* mxfp4_linear_prequantized: the oracle's GEMM tolerance, and bitwise the
  result of mxfp4_gemm_a4w4 on the same values in the GEMM layouts through
  the same kernel (small-M kernel reading the row-major operands directly
  for M <= 64, in either of its forms, and once per 64 rows up to 256 rows
  on few columns, except above 32 rows per launch on long K; permutation
  into the workspace, then the GEMM kernel, otherwise)."""

import numpy as np
import pytest
import torch

import mxfp4_block_scaled_quant_amd as mx
from mxfp4_block_scaled_quant_amd import inputs
from oracle import layout as L
from oracle import quant as Q
from tests.helpers import dev_bf16, host_u8, need_gpu
from tests.test_gpu_gemm import _check

pytestmark = pytest.mark.gpu


def _strided_u8(a, pad):
    """Device uint8 copy of the 2-D array `a` inside rows padded by `pad` bytes."""
    rows, cols = a.shape
    buf = np.zeros((rows, cols + pad), dtype=np.uint8)
    buf[:, :cols] = a
    return torch.from_numpy(buf).cuda()[:, :cols]


@pytest.mark.parametrize("rows,K,pad", [(1, 32, 0), (37, 4128, 3), (300, 256, 0), (64, 14336, 16),
                                        (17, 640, 1)])
def test_shuffle_scales_bit_exact(rows, K, pad):
    need_gpu()
    x = inputs.activations(rows, K, 5, edge=True)
    _, s = Q.quant_1x32(x)
    out = mx.mxfp4_shuffle_scales(_strided_u8(s, pad), rows, K)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(out), L.scales_to_gemm_layout(s))


CASES = [
    # name, M, N, K, kwargs, (ldq pad, lds pad)
    ("m1_1024x5120", 1, 1024, 5120, dict(seed=0, outliers=True), (0, 0)),         # 16-byte scale loads
    ("m16_1024x5120", 16, 1024, 5120, dict(seed=1, outliers=True, with_bias=True), (16, 16)),
    ("m37_300x2048_lds8", 37, 300, 2048, dict(seed=2), (0, 8)),                   # byte loads (lds % 16)
    ("m64_96x2048_lds16", 64, 96, 2048, dict(seed=3, with_bias=True), (32, 16)),
    ("m5_17x96", 5, 17, 96, dict(seed=9, with_bias=True), (16, 1)),
    ("m16_520x1056_bias", 16, 520, 1056, dict(seed=6, outliers=True, with_bias=True), (0, 0)),
    ("m37_96x4128_edge", 37, 96, 4128, dict(seed=5, edge=True, with_bias=True), (32, 5)),
    ("m64_300x640", 64, 300, 640, dict(seed=6, with_bias=True), (0, 0)),
    ("m65_257x2080", 65, 257, 2080, dict(seed=10, outliers=True), (16, 2)),      # 64 rows per launch
    ("m300_128x256_edge", 300, 128, 256, dict(seed=5, edge=True), (0, 0)),
    # one row tile, K > 8192: two strips and two groups per round past one
    # round of compute units (the byte scale loads even where the 16-byte
    # ones would be allowed), one strip and four groups per round within one
    ("m5_5120x8704_bias", 5, 5120, 8704, dict(seed=12, outliers=True, with_bias=True), (0, 0)),
    ("m16_1000x8704", 16, 1000, 8704, dict(seed=13, with_bias=True), (0, 0)),
    ("m9_1000x8704_pad", 9, 1000, 8704, dict(seed=13, with_bias=True), (16, 1)),
    ("m40_300x10240", 40, 300, 10240, dict(seed=14, outliers=True, with_bias=True), (16, 16)),
    ("m64_96x14336_pad", 64, 96, 14336, dict(seed=15, with_bias=True), (0, 3)),
    ("m129_1000x4128_pad", 129, 1000, 4128, dict(seed=16, outliers=True, with_bias=True), (16, 5)),  # 64 rows per launch
    ("m200_4200x1056_pad", 200, 4200, 1056, dict(seed=18, with_bias=True), (16, 3)),  # tiled path
    ("m128_8192x1056", 128, 8192, 1056, dict(seed=17, with_bias=True), (0, 0)),  # 64 rows per launch
    ("m100_2000x8704_pad", 100, 2000, 8704, dict(seed=19, with_bias=True), (16, 3)),  # permuted, 64 rows per launch
]


@pytest.mark.parametrize("name,M,N,K,kw,pads", CASES, ids=[c[0] for c in CASES])
def test_linear_prequantized(name, M, N, K, kw, pads):
    need_gpu()
    prob = inputs.linear_problem(M, N, K, **kw)
    W = mx.quantize_weight(dev_bf16(prob["w"]))
    q_rm, s_rm = Q.quant_1x32(prob["x"])                 # the producer's output (oracle bytes)
    xq, xs = _strided_u8(q_rm, pads[0]), _strided_u8(s_rm, pads[1])
    b = None if prob["bias"] is None else dev_bf16(prob["bias"])
    y32 = mx.mxfp4_linear_prequantized(xq, xs, W.w_pre, W.ws_pre, N, b, torch.float32)
    y16 = mx.mxfp4_linear_prequantized(xq, xs, W.w_pre, W.ws_pre, N, b, torch.bfloat16)
    # the same values in the GEMM layouts through the same kernel (and plan)
    mx.set_gemm_path(1 if M <= 64 else 0)
    try:
        q, s = mx.mxfp4_quant_1x32(dev_bf16(prob["x"]), mx.MXFP4_LAYOUT_GEMM)
        r32 = mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.float32)
        r16 = mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.bfloat16)
    finally:
        mx.set_gemm_path(0)
    torch.cuda.synchronize()
    y32n, r32n = y32.cpu().numpy(), r32.cpu().numpy()
    assert np.array_equal(y32n.view(np.uint32), r32n.view(np.uint32))
    assert torch.equal(y16.cpu().view(torch.int16), r16.cpu().view(torch.int16))
    _check(prob, y32n, y16.cpu().view(torch.int16).numpy().view(np.uint16))


PERSIST = [
    # name, M, N, K, (ldq pad, lds pad)
    ("m1_1040x4128", 1, 1040, 4128, (0, 0)),                  # ragged K tile, byte scale loads
    ("m5_300x640_pad", 5, 300, 640, (16, 1)),
    ("m16_5000x5120", 16, 5000, 5120, (0, 0)),                # 16-byte scale loads
    ("m33_520x1056_pad", 33, 520, 1056, (32, 3)),
    ("m48_4200x4096", 48, 4200, 4096, (16, 16)),
    ("m64_2064x6144", 64, 2064, 6144, (0, 0)),
    ("m16_24576x5120", 16, 24576, 5120, (0, 0)),              # chosen by default (six strips per CU)
    ("m40_12288x5120_pad", 40, 12288, 5120, (16, 16)),        # chosen by default (three per CU)
]


@pytest.mark.parametrize("name,M,N,K,pads", PERSIST, ids=[c[0] for c in PERSIST])
def test_linear_prequantized_persistent_form(name, M, N, K, pads):
    # The small-M kernel's persistent form reading the row-major operands:
    # bitwise what the same form computes from the GEMM layouts, and bitwise
    # the one-workgroup-per-strip form where both split K the same way; the
    # default choice is bitwise one of the two forms; the oracle bar on
    # sampled columns at the wide shapes.
    need_gpu()
    from tests.test_gpu_gemm import _same_k_split, _sample
    prob = inputs.linear_problem(M, N, K, 21, outliers=True, with_bias=True)
    W = mx.quantize_weight(dev_bf16(prob["w"]))
    q_rm, s_rm = Q.quant_1x32(prob["x"])
    xq, xs = _strided_u8(q_rm, pads[0]), _strided_u8(s_rm, pads[1])
    b = dev_bf16(prob["bias"])
    q, s = mx.mxfp4_quant_1x32(dev_bf16(prob["x"]), mx.MXFP4_LAYOUT_GEMM)
    res = {}
    try:
        for path in (0, 7, 8):
            mx.set_gemm_path(path)
            res[path] = (mx.mxfp4_linear_prequantized(xq, xs, W.w_pre, W.ws_pre, N, b, torch.float32),
                         mx.mxfp4_linear_prequantized(xq, xs, W.w_pre, W.ws_pre, N, b, torch.bfloat16))
        mx.set_gemm_path(7)
        r32 = mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.float32)
    finally:
        mx.set_gemm_path(0)
    torch.cuda.synchronize()
    y32 = res[7][0].cpu().numpy()
    assert np.array_equal(y32.view(np.uint32), r32.cpu().numpy().view(np.uint32))
    if _same_k_split(M, K):
        assert np.array_equal(y32.view(np.uint32), res[8][0].cpu().numpy().view(np.uint32))
        assert torch.equal(res[7][1].cpu().view(torch.int16), res[8][1].cpu().view(torch.int16))
    d32 = res[0][0].cpu().numpy().view(np.uint32)
    assert any(np.array_equal(d32, res[f][0].cpu().numpy().view(np.uint32)) for f in (7, 8))
    _check(prob, y32, res[7][1].cpu().view(torch.int16).numpy().view(np.uint16),
           cols=_sample(N, 96, N) if N > 4096 else None)


WIDE_K = [
    # name, M, N, K, (data, scale) row padding: more than 16 scale groups on
    # more strips than compute units, so each wave of the streaming form
    # loads its groups one per round over several rounds
    ("m1_4112x9216_lds3", 1, 4112, 9216, (0, 3)),          # byte scale loads
    ("m16_4112x12800", 16, 4112, 12800, (0, 0)),           # 16-byte loads, 25 groups on 13 waves
    ("m4_5120x14336_pad", 4, 5120, 14336, (16, 16)),
    ("m24_4112x9216_pad", 24, 4112, 9216, (16, 1)),        # two row tiles, byte loads
]


@pytest.mark.parametrize("name,M,N,K,pads", WIDE_K, ids=[c[0] for c in WIDE_K])
def test_linear_prequantized_wide_k(name, M, N, K, pads):
    # bitwise the GEMM-layout path through the streaming form over every
    # output (the same K split and order), and the oracle bar on sampled
    # columns
    need_gpu()
    from tests.test_gpu_gemm import _sample
    prob = inputs.linear_problem(M, N, K, 22, outliers=True, with_bias=True)
    W = mx.quantize_weight(dev_bf16(prob["w"]))
    q_rm, s_rm = Q.quant_1x32(prob["x"])
    xq, xs = _strided_u8(q_rm, pads[0]), _strided_u8(s_rm, pads[1])
    b = dev_bf16(prob["bias"])
    y32 = mx.mxfp4_linear_prequantized(xq, xs, W.w_pre, W.ws_pre, N, b, torch.float32)
    y16 = mx.mxfp4_linear_prequantized(xq, xs, W.w_pre, W.ws_pre, N, b, torch.bfloat16)
    q, s = mx.mxfp4_quant_1x32(dev_bf16(prob["x"]), mx.MXFP4_LAYOUT_GEMM)
    mx.set_gemm_path(8)
    try:
        r32 = mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.float32)
        r16 = mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.bfloat16)
    finally:
        mx.set_gemm_path(0)
    torch.cuda.synchronize()
    y32n = y32.cpu().numpy()
    assert np.array_equal(y32n.view(np.uint32), r32.cpu().numpy().view(np.uint32))
    assert torch.equal(y16.cpu().view(torch.int16), r16.cpu().view(torch.int16))
    _check(prob, y32n, y16.cpu().view(torch.int16).numpy().view(np.uint16), cols=_sample(N, 96, N))
