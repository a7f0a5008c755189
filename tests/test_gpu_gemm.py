"""GPU parity: the W4A4 linear (quant -> mxfp4_gemm_a4w4) against the oracle.

Bar: before the bf16 cast (fp32 output) |y - y_ref| <= 2^-18 (sum|a_i b_i| +
|bias|) per element; after the cast within 1 bf16 ulp of the rounded oracle,
or, where cancellation makes the pre-cast band wider than that, the rounding
of a value inside the band; the bf16 output equals the RNE of the kernel's
fp32 result; no NaN; identical bytes run to run.  Small shapes are checked
element by element, through the small-M kernel, the tiled kernel on its
own plan and at each output-tile width (256 and 128 columns) forced, each
also with its split-K schedule forced (every tile cut into K slices), and
the small-M kernel's persistent form (bitwise its streaming form where the
two split K alike); the full decode / prefill sweeps at sampled rows and columns (the
oracle quantises only the sampled rows of A and W, which is exact since
quantisation is per row)."""

import numpy as np
import pytest
import torch

import mxfp4_block_scaled_quant_amd as mx
from mxfp4_block_scaled_quant_amd import inputs
from oracle import formats as F
from oracle import linalg as G
from oracle import quant as Q
from tests.helpers import (check_bf16_cast, check_f32_tolerance, dev_bf16, host_bf16_bits,
                           need_gpu, tolerance_bound)

pytestmark = pytest.mark.gpu


def _run(prob, path, weight=None):
    x = dev_bf16(prob["x"])
    M, K = prob["x"].shape
    N = prob["w"].shape[0]
    W = weight if weight is not None else mx.quantize_weight(dev_bf16(prob["w"]))
    b = dev_bf16(prob["bias"]) if prob["bias"] is not None else None
    mx.set_gemm_path(path)
    try:
        q, s = mx.mxfp4_quant_1x32(x, mx.MXFP4_LAYOUT_GEMM)
        need = mx.gemm_workspace_bytes(M, N, K)
        ws = [torch.empty(need, dtype=torch.uint8, device="cuda") if need else None for _ in range(2)]
        y32 = mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.float32, workspace=ws[0])
        y16 = mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, torch.bfloat16, workspace=ws[1])
    finally:
        mx.set_gemm_path(0)
    torch.cuda.synchronize()
    assert_no_giveup(*ws)
    return y32.cpu().numpy(), host_bf16_bits(y16)


def assert_no_giveup(*workspaces):
    """After a split-schedule call, the first word of its workspace is
    nonzero only if a bounded wait for another slice gave up."""
    for ws in workspaces:
        if ws is not None:
            assert int(ws[:4].view(torch.int32).item()) == 0, "split schedule: a bounded wait gave up"


def _check(prob, y32, y16, rows=None, cols=None):
    x = prob["x"] if rows is None else prob["x"][rows]
    w = prob["w"] if cols is None else prob["w"][cols]
    bias = prob["bias"]
    if bias is not None and cols is not None:
        bias = bias[cols]
    y_ref, S = G.gemm_a4w4(x, w, bias)
    if rows is not None:
        y32, y16 = y32[rows], y16[rows]
    if cols is not None:
        y32, y16 = y32[:, cols], y16[:, cols]
    babs = None if bias is None else np.abs(F.bf16_to_f64(bias))[None, :]
    worst = check_f32_tolerance(y32, y_ref, S, babs)
    check_bf16_cast(y16, y_ref, tolerance_bound(S, babs))
    # the bf16 output is the single RNE cast of the kernel's own fp32 result
    assert np.array_equal(y16, G.to_bf16(y32.astype(np.float64)))
    return worst


SMALL = [
    # name, M, N, K, problem kwargs
    ("linear_16x1024x5120", 16, 1024, 5120, dict(seed=0, outliers=True)),
    ("edge_37x96x4128", 37, 96, 4128, dict(seed=5, edge=True)),
    ("edge_37x96x4128_bias", 37, 96, 4128, dict(seed=5, edge=True, with_bias=True)),
    ("edge_300x128x256", 300, 128, 256, dict(seed=5, edge=True)),
    ("edge_300x128x256_bias", 300, 128, 256, dict(seed=5, edge=True, with_bias=True)),
    ("tiles_300x520x1056", 300, 520, 1056, dict(seed=6, outliers=True, with_bias=True)),
    ("decode_64x300x640", 64, 300, 640, dict(seed=6, with_bias=True)),
    ("tiny_1x16x32", 1, 16, 32, dict(seed=9)),
    ("tiny_5x17x96", 5, 17, 96, dict(seed=9, with_bias=True)),
    ("ragged_257x257x2080", 257, 257, 2080, dict(seed=10, outliers=True)),
    # one row tile, more than 16 scale groups, every strip in one round of
    # compute units: one strip and four groups per wave in the small-M kernel
    ("widek_5x1000x8704", 5, 1000, 8704, dict(seed=14, outliers=True, with_bias=True)),
    ("widek_16x272x14336", 16, 272, 14336, dict(seed=15, with_bias=True)),
    # more row tiles there: four groups per round at two tiles, two at three
    # and four (ragged last round, ragged last scale group)
    ("widek_20x272x8192", 20, 272, 8192, dict(seed=16, outliers=True)),
    ("widek_40x300x10272", 40, 300, 10272, dict(seed=17, with_bias=True)),
    ("widek_64x96x14336_bias", 64, 96, 14336, dict(seed=18, edge=True, with_bias=True)),
    # past one round of compute units in strips, K <= 2048: one strip per
    # workgroup at one and four row tiles, two at two
    ("smallk_3x4200x2048", 3, 4200, 2048, dict(seed=19, with_bias=True)),
    ("smallk_64x4200x1056", 64, 4200, 1056, dict(seed=20, outliers=True)),
    ("smallk_30x4200x2048", 30, 4200, 2048, dict(seed=21, with_bias=True)),
]


@pytest.mark.parametrize("path", [1, 2, 3, 4, 5, 6],
                         ids=["smallM", "tiled", "tiled256", "tiled_split", "tiled128", "tiled128_split"])
@pytest.mark.parametrize("name,M,N,K,kw", SMALL, ids=[c[0] for c in SMALL])
def test_linear_small_shapes(name, M, N, K, kw, path):
    need_gpu()
    if path == 1 and M > 64:
        pytest.skip("the small-M kernel covers M <= 64")
    prob = inputs.linear_problem(M, N, K, **kw)
    y32, y16 = _run(prob, path)
    _check(prob, y32, y16)


@pytest.mark.parametrize("M", [17, 32, 33, 48, 49, 63, 65, 128, 129, 193, 256])
def test_linear_row_boundaries(M):
    # The automatic kernel choice on each side of its row boundaries: each
    # row-tile count (16 rows) of the small-M kernel up to 64 rows, then (on
    # these few columns) the small-M kernel once per 64 rows up to 256 rows
    # (257 rows, the large-M kernel, is a small-shape case above); 17 strips
    # of 16 columns, a ragged last scale group and a ragged last K-step.
    need_gpu()
    prob = inputs.linear_problem(M, 272, 1056, 11, outliers=True, with_bias=True)
    y32, y16 = _run(prob, 0)
    _check(prob, y32, y16)


@pytest.mark.parametrize("M,K", [(16, 8192), (32, 4096), (48, 4096), (64, 6144)])
def test_decode_widest_wave_split(M, K):
    # The small-M kernel at its most waves per workgroup for each row-tile
    # count (one 512-wide scale group per wave: 16, 8, 8 and 12 waves), its
    # largest LDS reduction; bf16 / fp32 output against the oracle, and the
    # MXFP4 output bitwise the quantisation of the bf16 output.
    need_gpu()
    N = 4128  # past one round of compute units in strips: two per workgroup
    prob = inputs.linear_problem(M, N, K, 12, outliers=True, with_bias=True)
    y32, y16 = _run(prob, 0)
    _check(prob, y32, y16)
    W = mx.quantize_weight(dev_bf16(prob["w"]))
    q, s = mx.mxfp4_quant_1x32(dev_bf16(prob["x"]), mx.MXFP4_LAYOUT_GEMM)
    oq, os_ = mx.mxfp4_gemm_a4w4_mxfp4_out(q, s, W.w_pre, W.ws_pre, M, N, K, dev_bf16(prob["bias"]))
    torch.cuda.synchronize()
    q_ref, s_ref = Q.quant_1x32(y16)
    assert np.array_equal(oq.cpu().numpy(), q_ref)
    assert np.array_equal(os_.cpu().numpy(), s_ref)


PERSIST = [
    # name, M, N, K: at most 12 scale groups (the persistent form applies);
    # fewer strips than compute units (one strip per workgroup), more (several,
    # a ragged last one), each row-tile count; at two and three row tiles
    # above 4096 of K the streaming form splits K differently
    ("1x1040x4128", 1, 1040, 4128),
    ("5x300x640", 5, 300, 640),
    ("16x5000x640", 16, 5000, 640),
    ("16x14336x5120", 16, 14336, 5120),
    ("33x520x1056", 33, 520, 1056),
    ("48x4200x4096", 48, 4200, 4096),
    ("32x24576x5120", 32, 24576, 5120),
    ("41x4100x6144", 41, 4100, 6144),
    ("64x2064x6144", 64, 2064, 6144),
    ("64x34816x5120", 64, 34816, 5120),
    # 13-24 groups at one or two row tiles: two groups per wave
    ("1x1040x8192", 1, 1040, 8192),
    ("9x17x6656", 9, 17, 6656),
    ("16x5000x12288", 16, 5000, 12288),
    ("20x2064x8704", 20, 2064, 8704),
    ("32x4100x7168", 32, 4100, 7168),
]


def _same_k_split(M, K):
    # the streaming form's groups per wave (at most 16 / 8 / 8 / 12 waves for
    # one to four row tiles) is that of the persistent form: one up to 12
    # groups, two for 13-24 groups at one or two row tiles (beyond that the
    # persistent form does not apply and both calls stream)
    mt = -(-M // 16)
    groups = -(-(-(-K // 128)) // 4)
    if groups <= 12:
        return groups <= (16 if mt == 1 else 12 if mt == 4 else 8)
    if groups > 24 or mt > 2:
        return True
    return groups > 16 if mt == 1 else groups <= 16


@pytest.mark.parametrize("name,M,N,K", PERSIST, ids=[c[0] for c in PERSIST])
def test_decode_persistent_form(name, M, N, K):
    # The small-M kernel's persistent form (one workgroup per compute unit
    # walking the strips, activations loaded once per wave) forced against
    # its one-workgroup-per-strip form: bitwise equal (fp32 and bf16 output,
    # with bias) where both split K the same way; within the oracle bar
    # (sampled columns at the wide shapes).
    need_gpu()
    prob = inputs.linear_problem(M, N, K, 13, outliers=True, with_bias=True)
    W = mx.quantize_weight(dev_bf16(prob["w"]))
    a = _run(prob, 7, weight=W)
    if _same_k_split(M, K):
        b = _run(prob, 8, weight=W)
        assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
        assert np.array_equal(a[1], b[1])
    _check(prob, *a, cols=_sample(N, 96, N) if N > 4096 else None)


def test_linear_deterministic():
    need_gpu()
    prob = inputs.linear_problem(300, 520, 1056, 6, outliers=True, with_bias=True)
    for path in (1, 2):
        p = dict(prob)
        if path == 1:
            p["x"] = prob["x"][:64]
        a = _run(p, path)
        b = _run(p, path)
        assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
        assert np.array_equal(a[1], b[1])


_WEIGHTS = {}


def _weight(N, K, seed):
    key = (N, K, seed)
    if key not in _WEIGHTS:
        _WEIGHTS.clear()
        w = inputs.weights(N, K, seed)
        _WEIGHTS[key] = (w, mx.quantize_weight(dev_bf16(w)))
    return _WEIGHTS[key]


NK = [(14336, 5120), (5120, 14336), (34816, 5120)]


def _sample(n, k, seed):
    r = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], r.choice(n, min(n, k), replace=False)]))


@pytest.mark.parametrize("N,K", NK, ids=[f"{n}x{k}" for n, k in NK])
def test_decode_sweep_full_size(N, K):
    # M in {1, 4, 16, 32, 64}, bias ~ N(0, 0.1), no outliers; the launch the
    # benchmark times (automatic kernel choice by M).
    need_gpu()
    w, W = _weight(N, K, 2)
    cols = _sample(N, 96, N)
    b = inputs.bias(N, 2)
    for M in (1, 4, 16, 32, 64):
        x = inputs.activations(M, K, 2)
        prob = {"x": x, "w": w, "bias": b}
        y32, y16 = _run(prob, 0, weight=W)
        _check(prob, y32, y16, cols=cols)


@pytest.mark.parametrize("M,N,K", [(16, 16400, 16384), (12, 16400, 15360)], ids=["16x16400x16384", "12x16400x15360"])
def test_decode_three_groups_per_wave(M, N, K):
    # 29-32 groups at 9-16 rows on many strips: three groups per wave; the
    # oracle bar on sampled columns
    need_gpu()
    w, W = _weight(N, K, 7)
    b = inputs.bias(N, 7)
    x = inputs.activations(M, K, 7, outliers=True)
    prob = {"x": x, "w": w, "bias": b}
    y32, y16 = _run(prob, 0, weight=W)
    _check(prob, y32, y16, cols=_sample(N, 96, N))


@pytest.mark.parametrize("M", [1, 16])
def test_decode_group_rounds_same_bits(M):
    # More than 16 scale groups at one row tile: with 513 strips (two-strip
    # workgroups filling a round of compute units) each wave loads its groups
    # one per round, with 320 strips two per round; the K split and order are
    # the same, so the first 5120 columns agree bitwise.  The oracle bar on
    # sampled columns of the wide product.
    need_gpu()
    N, K = 8208, 8704
    w, W = _weight(N, K, 4)
    b = inputs.bias(N, 4)
    x = inputs.activations(M, K, 4, outliers=True)
    prob = {"x": x, "w": w, "bias": b}
    y32, y16 = _run(prob, 0, weight=W)
    part = {"x": x, "w": w[:5120], "bias": b[:5120]}
    p32, p16 = _run(part, 0)
    assert np.array_equal(y32[:, :5120].view(np.uint32), p32.view(np.uint32))
    assert np.array_equal(y16[:, :5120], p16)
    _check(prob, y32, y16, cols=_sample(N, 96, N))


ROWS = [
    # M, N, K, bias: up to 256 rows on few columns (ceil(M/64) * N <= 16384)
    # run the small-M kernel once per 64 rows
    (65, 4096, 4096, False),
    (100, 1000, 5120, True),
    (128, 8192, 8192, True),
    (192, 4096, 4128, True),
    (250, 2000, 1056, False),
]


@pytest.mark.parametrize("M,N,K,bias", ROWS, ids=[f"{m}x{n}x{k}" for m, n, k, _ in ROWS])
def test_gemm_rows_per_launch(M, N, K, bias):
    # bitwise the small-M kernel called on rows 0-63 and on the rest
    # separately, and the oracle bar (sampled columns at the widest)
    need_gpu()
    w, W = _weight(N, K, 6)
    b = inputs.bias(N, 6) if bias else None
    x = inputs.activations(M, K, 6, outliers=True)
    prob = {"x": x, "w": w, "bias": b}
    y32, y16 = _run(prob, 0, weight=W)
    for r0 in range(0, M, 64):
        part = {"x": x[r0:r0 + 64], "w": w, "bias": b}
        p32, p16 = _run(part, 0, weight=W)
        assert np.array_equal(y32[r0:r0 + 64].view(np.uint32), p32.view(np.uint32)), r0
        assert np.array_equal(y16[r0:r0 + 64], p16), r0
    _check(prob, y32, y16, cols=_sample(N, 96, N) if N > 4096 else None)


@pytest.mark.parametrize("N,K", NK, ids=[f"{n}x{k}" for n, k in NK])
def test_prefill_sweep_full_size(N, K):
    # M in {512, 2048, 8192}, 1% outlier channels x20, no bias.
    need_gpu()
    w, W = _weight(N, K, 3)
    cols = _sample(N, 64, N + 1)
    for M in (512, 2048, 8192):
        x = inputs.activations(M, K, 3, outliers=True)
        prob = {"x": x, "w": w, "bias": None}
        y32, y16 = _run(prob, 0, weight=W)
        rows = _sample(M, 64, M)
        _check(prob, y32, y16, rows=rows, cols=cols)


@pytest.mark.parametrize("path,K", [(1, 64), (3, 192), (5, 192)], ids=["smallM", "tiled256", "tiled128"])
def test_gemm_weight_scales_exact(path, K):
    # Every weight scale byte 0..254 with every E2M1 code, times identity
    # activations (each row one 1.0: quantised exactly, code 6 at scale 125),
    # so out[m, n] is the single nonzero product dq(W)[n, m]: exact in fp32
    # (values past the fp32 range are infinite on both sides) and in bf16.
    # Zeros compare without their sign (the sum of the other, zero, products
    # decides it).
    need_gpu()
    N = 512
    nb = K // 32
    n_idx = np.arange(N)[:, None]
    scales = ((n_idx * nb + np.arange(nb)[None, :]) % 255).astype(np.uint8)
    codes = ((np.arange(K)[None, :] + n_idx) % 16).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    w_pre, ws_pre = mx.mxfp4_preshuffle_weight(torch.from_numpy(packed).cuda(),
                                               torch.from_numpy(scales).cuda(), N, K)
    eye = np.zeros((K, K), dtype=np.uint16)
    eye[np.arange(K), np.arange(K)] = 0x3F80
    mx.set_gemm_path(path)
    try:
        q, s = mx.mxfp4_quant_1x32(dev_bf16(eye), mx.MXFP4_LAYOUT_GEMM)
        y32 = mx.mxfp4_gemm_a4w4(q, s, w_pre, ws_pre, K, N, K, None, torch.float32)
        y16 = mx.mxfp4_gemm_a4w4(q, s, w_pre, ws_pre, K, N, K, None, torch.bfloat16)
    finally:
        mx.set_gemm_path(0)
    torch.cuda.synchronize()
    from oracle import quant as Q
    dq = Q.dequant(packed, scales)
    with np.errstate(over="ignore"):
        assert np.array_equal(y32.cpu().numpy(), dq.T.astype(np.float32))      # -0.0 == 0.0, inf == inf
    unsigned_zero = lambda b: np.where((b & 0x7FFF) == 0, 0, b)
    assert np.array_equal(unsigned_zero(host_bf16_bits(y16)), unsigned_zero(F.f64_to_bf16(dq.T)))


@pytest.mark.parametrize("path", [1, 2, 3, 4, 5, 6],
                         ids=["smallM", "tiled", "tiled256", "tiled_split", "tiled128", "tiled128_split"])
@pytest.mark.parametrize("dtype,pad", [(torch.bfloat16, 8), (torch.bfloat16, 3), (torch.float32, 4),
                                       (torch.float32, 1)],
                         ids=["bf16_pad8", "bf16_pad3", "f32_pad4", "f32_pad1"])
def test_gemm_strided_output(path, dtype, pad):
    # out is a view with row stride N + pad inside a sentinel-filled buffer:
    # every output mode (16-byte row pieces, single elements; bf16 / fp32)
    # writes exactly the [M, N] window, bitwise as into a contiguous output.
    need_gpu()
    M = 37 if path == 1 else 300
    N, K = 96, 4128
    prob = inputs.linear_problem(M, N, K, 5, edge=True, with_bias=True)
    W = mx.quantize_weight(dev_bf16(prob["w"]))
    b = dev_bf16(prob["bias"])
    q, s = mx.mxfp4_quant_1x32(dev_bf16(prob["x"]), mx.MXFP4_LAYOUT_GEMM)
    buf = torch.full((M, N + pad), -7.0, dtype=dtype, device="cuda")
    mx.set_gemm_path(path)
    try:
        ref = mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, dtype)
        mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, b, dtype, out=buf[:, :N])
        lin = torch.full((M, N + pad), -7.0, dtype=dtype, device="cuda")
        mx.mxfp4_linear(dev_bf16(prob["x"]), W.w_pre, W.ws_pre, N, b, dtype, out=lin[:, :N])
        # the fp32 and bf16 results the oracle check pairs, on the same schedule
        lin32 = mx.mxfp4_linear(dev_bf16(prob["x"]), W.w_pre, W.ws_pre, N, b, torch.float32)
        lin16 = (lin[:, :N].contiguous() if dtype == torch.bfloat16 else
                 mx.mxfp4_linear(dev_bf16(prob["x"]), W.w_pre, W.ws_pre, N, b, torch.bfloat16))
    finally:
        mx.set_gemm_path(0)
    torch.cuda.synchronize()
    iview = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(buf[:, :N].contiguous().view(iview), ref.view(iview))
    assert torch.all(buf[:, N:] == -7.0)
    assert torch.all(lin[:, N:] == -7.0)
    _check(prob, lin32.cpu().numpy(), host_bf16_bits(lin16))
