"""GPU parity of mxfp4_linear: bf16 activations -> per-1x32 quantisation ->
FP4 GEMM (+ bias) in one call, the quantisation fused into the GEMM kernel
for M <= 4 (the streaming small-M form, or its persistent form on wide N)
and done through a workspace above that; the persistent form's fusion is
also forced at M <= 32 (one or two row tiles).

Bars: the oracle's GEMM tolerance (as for mxfp4_gemm_a4w4); the output is
bitwise that of mxfp4_quant_1x32 followed by the small-M mxfp4_gemm_a4w4 up
to M = 64 wherever the two share their K split (all but the fused kernel
at K > 8192, which splits K over fewer waves); and the fused encoder
reproduces the oracle's quantisation exactly for every finite bf16 value."""

import numpy as np
import pytest
import torch

import mxfp4_block_scaled_quant_amd as mx
from mxfp4_block_scaled_quant_amd import inputs
from oracle import formats as F
from oracle import quant as Q
from tests.helpers import dev_bf16, host_bf16_bits, need_gpu
from tests.test_gpu_gemm import NK, _check, _sample, _weight

pytestmark = pytest.mark.gpu


def _linear(x_bits, W, N, bias_bits, ldx_pad=0):
    M, K = x_bits.shape
    if ldx_pad:
        buf = np.zeros((M, K + ldx_pad), dtype=np.uint16)
        buf[:, :K] = x_bits
        x = dev_bf16(buf)[:, :K]
    else:
        x = dev_bf16(x_bits)
    b = None if bias_bits is None else dev_bf16(bias_bits)
    y32 = mx.mxfp4_linear(x, W.w_pre, W.ws_pre, N, b, torch.float32)
    y16 = mx.mxfp4_linear(x, W.w_pre, W.ws_pre, N, b, torch.bfloat16)
    torch.cuda.synchronize()
    return y32.cpu().numpy(), host_bf16_bits(y16)


def _same_split(M, N, K):
    """The fused kernel (M = 1; M = 2 at K <= 16384; M <= 4 at N < 16384,
    K <= 8192, except M >= 3 at 8192 < N <= 12288; M <= 4 at N <= 4096,
    K <= 16384) splits K like the small-M GEMM except beyond 16 scale
    groups (K > 8192)."""
    wide_k = K <= 16384 and (M == 2 or N <= 4096)
    fused = M == 1 or (M <= 4 and N < 16384 and not (M >= 3 and 8192 < N <= 12288)
                       and (K <= 8192 or wide_k)) or (M == 2 and K <= 16384)
    groups = -(-(-(-K // 128)) // 4)
    return not (fused and groups > 16)


def _two_launch(x_bits, W, N, bias_bits):
    M, K = x_bits.shape
    b = None if bias_bits is None else dev_bf16(bias_bits)
    mx.set_gemm_path(1)
    try:
        q, s = mx.mxfp4_quant_1x32(dev_bf16(x_bits), mx.MXFP4_LAYOUT_GEMM)
        y32 = mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.float32)
        y16 = mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.bfloat16)
    finally:
        mx.set_gemm_path(0)
    torch.cuda.synchronize()
    return y32.cpu().numpy(), host_bf16_bits(y16)


CASES = [
    # name, M, N, K, problem kwargs, ldx padding (fused quantisation at M = 1,
    # at M <= 4 for N < 16384, K <= 8192, and up to K = 16384 at M = 2 or
    # N <= 4096; else through the workspace)
    ("m1_1024x5120", 1, 1024, 5120, dict(seed=0, outliers=True), 0),
    ("m2_96x4128_edge", 2, 96, 4128, dict(seed=5, edge=True), 16),
    ("m1_1056x14336_bias", 1, 1056, 14336, dict(seed=4, with_bias=True), 0),    # fused, wide K
    ("m3_1056x14336_bias", 3, 1056, 14336, dict(seed=4, with_bias=True), 0),   # fused, two rounds
    ("m2_2000x16384_bias", 2, 2000, 16384, dict(seed=12, with_bias=True), 0),   # fused, 32 groups
    ("m4_1000x10240_edge", 4, 1000, 10240, dict(seed=13, edge=True), 16),      # fused, ragged rounds
    ("m3_4112x9216", 3, 4112, 9216, dict(seed=14, outliers=True), 0),          # workspace (N > 4096)
    ("m1_17x8320", 1, 17, 8320, dict(seed=11, outliers=True), 8),               # fused, 17 groups
    ("m4_300x640_bias", 4, 300, 640, dict(seed=6, with_bias=True), 0),
    ("m4_16x32", 4, 16, 32, dict(seed=9), 8),
    ("m5_17x96", 5, 17, 96, dict(seed=9, with_bias=True), 8),
    ("m15_96x4128_edge", 15, 96, 4128, dict(seed=5, edge=True), 24),
    ("m16_1024x5120", 16, 1024, 5120, dict(seed=0, outliers=True), 0),
    ("m16_520x1056_bias", 16, 520, 1056, dict(seed=6, outliers=True, with_bias=True), 0),
    ("m16_16x32", 16, 16, 32, dict(seed=9), 0),
    ("m17_257x2080", 17, 257, 2080, dict(seed=10, outliers=True), 0),      # workspace + small-M
    ("m37_96x4128_edge_bias", 37, 96, 4128, dict(seed=5, edge=True, with_bias=True), 8),
    ("m100_1000x5120_bias", 100, 1000, 5120, dict(seed=7, outliers=True, with_bias=True), 8),  # 64 rows per launch
    ("m200_96x1056", 200, 96, 1056, dict(seed=8, edge=True), 0),
    ("m300_520x1056_bias", 300, 520, 1056, dict(seed=6, outliers=True, with_bias=True), 0),  # tiled
]


@pytest.mark.parametrize("name,M,N,K,kw,pad", CASES, ids=[c[0] for c in CASES])
def test_linear_matches_oracle(name, M, N, K, kw, pad):
    need_gpu()
    prob = inputs.linear_problem(M, N, K, **kw)
    W = mx.quantize_weight(dev_bf16(prob["w"]))
    y32, y16 = _linear(prob["x"], W, N, prob["bias"], ldx_pad=pad)
    _check(prob, y32, y16)
    if M <= 64 and _same_split(M, N, K):
        # bitwise the two-call form through the small-M GEMM
        r32, r16 = _two_launch(prob["x"], W, N, prob["bias"])
        assert np.array_equal(y32.view(np.uint32), r32.view(np.uint32))
        assert np.array_equal(y16, r16)


def test_fused_encoding_every_bf16_value():
    # x holds every finite bf16 value (shuffled, 16 rows of 4096), passed to
    # the fused kernel 4 rows at a time; the weight is the identity (each row
    # one 1.0: code 6 at scale byte 125, exactly 1.0), so out[m, n] is the
    # single product dq(Q(x))[m, n]: exact in fp32.  Zeros compare without
    # their sign (the sum of the other, zero, products decides it).
    need_gpu()
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = u[(u & 0x7F80) != 0x7F80]
    rng = np.random.default_rng(7)
    K = 4096
    vals = np.concatenate([rng.permutation(finite), np.zeros(16 * K - finite.size, np.uint16)])
    x = vals.reshape(16, K)
    eye = np.zeros((K, K), dtype=np.uint16)
    eye[np.arange(K), np.arange(K)] = 0x3F80
    W = mx.quantize_weight(dev_bf16(eye))
    packed, scales = Q.quant_1x32(x)
    dq = Q.dequant(packed, scales).astype(np.float32)
    unsigned = lambda a: np.where(a == 0, np.float32(0), a)
    for r0, M in [(0, 4), (4, 4), (8, 4), (12, 4), (3, 1), (5, 2), (9, 3)]:
        y32, _ = _linear(x[r0:r0 + M], W, K, None)
        assert np.array_equal(unsigned(y32), unsigned(dq[r0:r0 + M])), (r0, M)


@pytest.mark.parametrize("N,K", NK, ids=[f"{n}x{k}" for n, k in NK])
def test_linear_decode_full_size(N, K):
    # The benchmark's launch at M in {1, 4, 16} (bias ~ N(0, 0.1)): bitwise the
    # two-call form over every output, and the oracle at sampled columns.
    need_gpu()
    w, W = _weight(N, K, 2)
    cols = _sample(N, 96, N)
    b = inputs.bias(N, 2)
    for M in (1, 4, 16):
        x = inputs.activations(M, K, 2)
        y32, y16 = _linear(x, W, N, b)
        if _same_split(M, N, K):
            r32, r16 = _two_launch(x, W, N, b)
            assert np.array_equal(y32.view(np.uint32), r32.view(np.uint32))
            assert np.array_equal(y16, r16)
        _check({"x": x, "w": w, "bias": b}, y32, y16, cols=cols)


def test_linear_deterministic_and_empty():
    need_gpu()
    prob = inputs.linear_problem(16, 520, 1056, 6, outliers=True, with_bias=True)
    W = mx.quantize_weight(dev_bf16(prob["w"]))
    a = _linear(prob["x"], W, 520, prob["bias"])
    b = _linear(prob["x"], W, 520, prob["bias"])
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32)) and np.array_equal(a[1], b[1])
    empty = mx.mxfp4_linear(torch.empty((0, 1056), dtype=torch.bfloat16, device="cuda"),
                            W.w_pre, W.ws_pre, 520)
    assert empty.shape == (0, 520)


PERSIST = [
    # name, M, N, K, problem kwargs, ldx padding: the quantisation fused into
    # the small-M kernel's persistent form (M <= 32, at most 12 scale groups)
    ("m1_1024x5120", 1, 1024, 5120, dict(seed=0, outliers=True), 0),
    ("m2_96x4128_edge", 2, 96, 4128, dict(seed=5, edge=True), 16),       # ragged K tile
    ("m5_17x96_bias", 5, 17, 96, dict(seed=9, with_bias=True), 8),
    ("m8_300x640_bias", 8, 300, 640, dict(seed=6, with_bias=True), 0),
    ("m15_520x1056_edge", 15, 520, 1056, dict(seed=5, edge=True), 24),
    ("m16_5000x6144_bias", 16, 5000, 6144, dict(seed=3, outliers=True, with_bias=True), 0),  # 12 groups
    ("m16_34816x5120", 16, 34816, 5120, dict(seed=2, with_bias=True), 0),
    # two row tiles
    ("m17_300x640_bias", 17, 300, 640, dict(seed=6, with_bias=True), 8),
    ("m24_520x4128_edge", 24, 520, 4128, dict(seed=5, edge=True), 16),   # 9 groups, ragged K tile
    ("m31_96x1056_edge", 31, 96, 1056, dict(seed=4, edge=True), 24),
    ("m32_5000x6144_bias", 32, 5000, 6144, dict(seed=3, outliers=True, with_bias=True), 0),  # 12 groups
    ("m32_14336x4096", 32, 14336, 4096, dict(seed=1, with_bias=True), 0),
]


@pytest.mark.parametrize("name,M,N,K,kw,pad", PERSIST, ids=[c[0] for c in PERSIST])
def test_linear_persistent_form(name, M, N, K, kw, pad):
    # mxfp4_linear with the quantisation inside the persistent form (forced):
    # bitwise quantisation + the persistent GEMM and quantisation + the
    # one-workgroup-per-strip GEMM (one group per wave in both; the latter
    # only while it keeps one group per wave: at two row tiles up to 8
    # groups), and the oracle bar (sampled columns at the widest shape).
    need_gpu()
    G = -(-(-(-K // 128)) // 4)
    prob = inputs.linear_problem(M, N, K, **kw)
    W = mx.quantize_weight(dev_bf16(prob["w"]))
    mx.set_gemm_path(7)
    try:
        y32, y16 = _linear(prob["x"], W, N, prob["bias"], ldx_pad=pad)
    finally:
        mx.set_gemm_path(0)
    for path in ((7, 8) if M <= 16 or G <= 8 else (7,)):
        b = None if prob["bias"] is None else dev_bf16(prob["bias"])
        mx.set_gemm_path(path)
        try:
            q, s = mx.mxfp4_quant_1x32(dev_bf16(prob["x"]), mx.MXFP4_LAYOUT_GEMM)
            r32 = mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.float32)
            r16 = mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.bfloat16)
        finally:
            mx.set_gemm_path(0)
        torch.cuda.synchronize()
        assert np.array_equal(y32.view(np.uint32), r32.cpu().numpy().view(np.uint32)), path
        assert np.array_equal(y16, host_bf16_bits(r16)), path
    _check(prob, y32, y16, cols=_sample(N, 96, N) if N > 4096 else None)


def test_persistent_encoding_every_bf16_value():
    # As the fused-encoding test above, through the persistent form's encoder
    # (forced), 32, 20, 16, 5 and 1 rows at a time (every finite value in
    # each 16-row half).
    need_gpu()
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = u[(u & 0x7F80) != 0x7F80]
    rng = np.random.default_rng(8)
    K = 4096
    half = lambda: np.concatenate([rng.permutation(finite), np.zeros(16 * K - finite.size, np.uint16)])
    x = np.concatenate([half(), half()]).reshape(32, K)
    eye = np.zeros((K, K), dtype=np.uint16)
    eye[np.arange(K), np.arange(K)] = 0x3F80
    W = mx.quantize_weight(dev_bf16(eye))
    packed, scales = Q.quant_1x32(x)
    dq = Q.dequant(packed, scales).astype(np.float32)
    unsigned = lambda a: np.where(a == 0, np.float32(0), a)
    mx.set_gemm_path(7)
    try:
        for r0, M in [(0, 32), (7, 20), (0, 16), (16, 16), (3, 5), (11, 5), (15, 1)]:
            y32, _ = _linear(x[r0:r0 + M], W, K, None)
            assert np.array_equal(unsigned(y32), unsigned(dq[r0:r0 + M])), (r0, M)
    finally:
        mx.set_gemm_path(0)


WIDE = [(1, 8208, 5120), (2, 10240, 8192), (3, 10240, 5120), (2, 16400, 4096), (2, 20480, 8704)]


@pytest.mark.parametrize("M,N,K", WIDE, ids=[f"m{m}_{n}x{k}" for m, n, k in WIDE])
def test_linear_wide_shapes(M, N, K):
    # Between two and three strips per compute unit the fused kernel runs one
    # strip per workgroup at M <= 2, and M >= 3 goes through quantisation +
    # GEMM; on many strips M = 2 is fused (past 16 groups with its own K
    # split): bitwise quantisation + GEMM where the K splits agree, and the
    # oracle bar on sampled columns.
    need_gpu()
    w, W = _weight(N, K, 5)
    b = inputs.bias(N, 5)
    x = inputs.activations(M, K, 5, outliers=True)
    y32, y16 = _linear(x, W, N, b)
    if _same_split(M, N, K):
        r32, r16 = _two_launch(x, W, N, b)
        assert np.array_equal(y32.view(np.uint32), r32.view(np.uint32))
        assert np.array_equal(y16, r16)
    _check({"x": x, "w": w, "bias": b}, y32, y16, cols=_sample(N, 96, N))
