"""GPU parity: a16wfp4_bmm against the oracle (MLA absorbed K-up / V-up on one
GPU's 16 heads, plus ragged shapes), both output layouts."""

import numpy as np
import pytest
import torch

import mxfp4_block_scaled_quant_amd as mx
from mxfp4_block_scaled_quant_amd import inputs
from oracle import linalg as G
from oracle import quant as Q
from tests.helpers import (check_bf16_cast, check_f32_tolerance, dev_bf16, host_bf16_bits,
                           need_gpu, tolerance_bound)

pytestmark = pytest.mark.gpu


def _run(prob, batch_major):
    B, M, K = prob["x"].shape
    N = prob["w"].shape[1]
    x = dev_bf16(prob["x"])
    W = mx.quantize_weight(dev_bf16(prob["w"]))
    y32 = mx.a16wfp4_bmm(x, W.w_pre, W.ws_pre, N, batch_major=batch_major, out_dtype=torch.float32)
    y16 = mx.a16wfp4_bmm(x, W.w_pre, W.ws_pre, N, batch_major=batch_major)
    torch.cuda.synchronize()
    y32, y16 = y32.cpu().numpy(), host_bf16_bits(y16)
    if batch_major:                      # [M, B, N] -> [B, M, N]
        y32, y16 = y32.transpose(1, 0, 2), y16.transpose(1, 0, 2)
    return y32, y16


def _check(prob, y32, y16, rows=None):
    x = prob["x"] if rows is None else prob["x"][:, rows]
    qw, sw = Q.quant_1x32(prob["w"])
    o, S = G.bmm_a16wfp4(x, qw, sw)
    if rows is not None:
        y32, y16 = y32[:, rows], y16[:, rows]
    check_f32_tolerance(y32, o, S)
    check_bf16_cast(y16, o, tolerance_bound(S))
    assert np.array_equal(y16, G.to_bf16(y32.astype(np.float64)))


CASES = [
    # name, B, M, N, K, batch_major
    ("kup_M1", 16, 1, 512, 192, False),
    ("kup_M64", 16, 64, 512, 192, False),
    ("kup_M256", 16, 256, 512, 192, False),
    ("vup_M1", 16, 1, 256, 512, True),
    ("vup_M64", 16, 64, 256, 512, True),
    ("vup_M256", 16, 256, 256, 512, True),
    ("ragged_3x37x96x160", 3, 37, 96, 160, False),
    ("colblocks_2x20x200x256", 2, 20, 200, 256, True),      # two column blocks, the last ragged
    ("colblocks_5x3x392x512", 5, 3, 392, 512, False),
    ("ragged_2x70x30x4128", 2, 70, 30, 4128, True),
    # 81 m-tiles over 16 workgroups per head: six per workgroup (the
    # three-stage ring), the last workgroup with three, the last tile 7 rows
    ("kup_M1287", 16, 1287, 512, 192, False),
    ("vup_M1287", 16, 1287, 256, 512, True),
    # the head's columns over two workgroups (a few m-tiles per head): K-up
    # with 32 m-tiles (four per workgroup, the last 4 rows), V-up with 10
    # (the last 6 rows)
    ("kup_M500_colsplit", 16, 500, 512, 192, False),
    ("vup_M150_colsplit", 16, 150, 256, 512, True),
]


@pytest.mark.parametrize("name,B,M,N,K,bm", CASES, ids=[c[0] for c in CASES])
def test_bmm(name, B, M, N, K, bm):
    need_gpu()
    prob = inputs.bmm_problem(B, M, N, K, 4)
    y32, y16 = _run(prob, bm)
    _check(prob, y32, y16)


@pytest.mark.parametrize("name,N,K,bm", [("kup_M4096", 512, 192, False), ("vup_M4096", 256, 512, True)])
def test_bmm_full_size_sampled_rows(name, N, K, bm):
    need_gpu()
    prob = inputs.bmm_problem(16, 4096, N, K, 4)
    y32, y16 = _run(prob, bm)
    rows = np.unique(np.concatenate([[0, 4095], np.random.default_rng(1).choice(4096, 62, replace=False)]))
    _check(prob, y32, y16, rows=rows)


def test_bmm_exact_mxfp4_activations_match_gemm():
    # Cross-path identity: activations that are MXFP4 numbers give the same
    # product through the BMM as through quant + W4A4 GEMM (within tolerance
    # of each other, both against the oracle).
    need_gpu()
    B, M, N, K = 4, 48, 64, 256
    prob = inputs.bmm_problem(B, M, N, K, 5)
    qx, sx = Q.quant_1x32(prob["x"])
    from oracle import formats as F
    prob["x"] = F.f64_to_bf16(Q.dequant(qx, sx))
    y32, _ = _run(prob, False)
    for b in range(B):
        W = mx.quantize_weight(dev_bf16(prob["w"][b]))
        q, s = mx.mxfp4_quant_1x32(dev_bf16(prob["x"][b]))
        g = mx.mxfp4_gemm_a4w4(q, s, W.w_pre, W.ws_pre, M, N, K, None, torch.float32).cpu().numpy()
        ref, S = G.gemm_a4w4_from_quant(qx[b], sx[b], *Q.quant_1x32(prob["w"][b]))
        check_f32_tolerance(g, ref, S)
        check_f32_tolerance(y32[b], ref, S)


def test_bmm_dequant_exact_every_scale():
    # Weight dequantisation, pinned element by element: one head (K-up shape,
    # the streaming kernel) whose blocks carry every scale byte 0..252 (every
    # scale quantisation of bf16 data can produce: amax < 2^128) and every
    # E2M1 code, times identity activations, so out[m, n] is the single
    # nonzero product 1 * dq(W)[n, m]: exact in fp32 and in bf16 (each such
    # dequantised value is a bf16 number).  Zeros compare without their sign
    # (the sum over the other, zero, products decides it).
    need_gpu()
    B, N, K = 1, 512, 192
    nb = K // 32
    n_idx = np.arange(N)[:, None]
    scales = ((n_idx * nb + np.arange(nb)[None, :]) % 253).astype(np.uint8)          # [N, K/32]
    codes = ((np.arange(K)[None, :] + n_idx) % 16).astype(np.uint8)                 # [N, K]
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)              # [N, K/2]
    w_pre, ws_pre = mx.mxfp4_preshuffle_weight(torch.from_numpy(packed).cuda(),
                                               torch.from_numpy(scales).cuda(), N, K, batch=B)
    eye = np.zeros((B, K, K), dtype=np.uint16)
    eye[0, np.arange(K), np.arange(K)] = 0x3F80                                        # bf16 1.0
    x = dev_bf16(eye)
    y32 = mx.a16wfp4_bmm(x, w_pre, ws_pre, N, out_dtype=torch.float32)
    y16 = mx.a16wfp4_bmm(x, w_pre, ws_pre, N)
    torch.cuda.synchronize()
    dq = Q.dequant(packed, scales)                                                  # fp64 [N, K]
    assert np.array_equal(y32.cpu().numpy()[0], dq.T.astype(np.float32))          # -0.0 == 0.0
    from oracle import formats as F
    unsigned_zero = lambda b: np.where((b & 0x7FFF) == 0, 0, b)
    assert np.array_equal(unsigned_zero(host_bf16_bits(y16)[0]), unsigned_zero(F.f64_to_bf16(dq.T)))


@pytest.mark.parametrize("name,B,M,N,K", [("kup_M37", 16, 37, 512, 192), ("vup_M70", 16, 70, 256, 512),
                                          ("small_M3", 4, 3, 200, 256), ("kup_M1287", 16, 1287, 512, 192)])
def test_bmm_strided_activations_and_output(name, B, M, N, K):
    # x as a view with padded rows and heads (sxm = K + 8, sxb = (M + 3) * sxm),
    # out as a view with padded rows inside a sentinel buffer: bitwise the
    # contiguous call, padding untouched.
    need_gpu()
    prob = inputs.bmm_problem(B, M, N, K, 7)
    W = mx.quantize_weight(dev_bf16(prob["w"]))
    big = np.zeros((B, M + 3, K + 8), dtype=np.uint16)
    big[:, :M, :K] = prob["x"]
    xs = dev_bf16(big)[:, :M, :K]
    ref = mx.a16wfp4_bmm(dev_bf16(prob["x"]), W.w_pre, W.ws_pre, N, out_dtype=torch.float32)
    ob = torch.full((B, M, N + 6), -7.0, dtype=torch.float32, device="cuda")   # row stride even (documented)
    mx.a16wfp4_bmm(xs, W.w_pre, W.ws_pre, N, out=ob[:, :, :N], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(ob[:, :, :N].contiguous().view(torch.int32), ref.view(torch.int32))
    assert torch.all(ob[:, :, N:] == -7.0)
    y16 = mx.a16wfp4_bmm(xs, W.w_pre, W.ws_pre, N)
    _check(prob, ref.cpu().numpy(), host_bf16_bits(y16))
