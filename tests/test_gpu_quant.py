"""GPU parity: mxfp4_quant_1x32 and mxfp4_preshuffle_weight against the oracle,
byte for byte (packed FP4, scales in both layouts, preshuffled weights)."""

import numpy as np
import pytest
import torch

import mxfp4_block_scaled_quant_amd as mx
from mxfp4_block_scaled_quant_amd import inputs
from oracle import formats as F
from oracle import layout as L
from oracle import quant as Q
from tests.helpers import dev_bf16, host_u8, need_gpu

pytestmark = pytest.mark.gpu

ACT_CASES = [
    # name, M, K, generator kwargs
    ("linear_16x5120_outliers", 16, 5120, dict(seed=0, outliers=True)),
    ("edge_37x4128", 37, 4128, dict(seed=5, edge=True)),
    ("edge_300x256", 300, 256, dict(seed=5, edge=True)),
    ("ragged_130x1056", 130, 1056, dict(seed=7, outliers=True)),
    ("single_block", 1, 32, dict(seed=8)),
    ("decode_64x14336", 64, 14336, dict(seed=2)),
]


def _gpu_quant(x_bits, layout, ldx_pad=0, ldq_pad=0):
    M, K = x_bits.shape
    if ldx_pad:
        wide = np.zeros((M, K + ldx_pad), dtype=np.uint16)
        wide[:, :K] = x_bits
        x = dev_bf16(wide)[:, :K]
    else:
        x = dev_bf16(x_bits)
    q = None
    if ldq_pad:
        q = torch.full((M, K // 2 + ldq_pad), 0xAB, dtype=torch.uint8, device="cuda")[:, :K // 2]
    elif layout == mx.MXFP4_LAYOUT_GEMM:
        # poison the output so every padding byte must be written
        q = torch.full((mx.data_bytes(M, K, layout),), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((mx.scale_bytes(M, K, layout),), 0xFF, dtype=torch.uint8, device="cuda")
    q, s = mx.mxfp4_quant_1x32(x, layout, q=q, scales=s)
    torch.cuda.synchronize()
    return host_u8(q), host_u8(s)


def _expect(x_bits, layout):
    q_ref, s_ref = Q.quant_1x32(x_bits)
    if layout == mx.MXFP4_LAYOUT_ROWMAJOR:
        return q_ref, s_ref.ravel()
    return L.to_gemm_layout(q_ref, s_ref)


@pytest.mark.parametrize("layout", [0, 1], ids=["rowmajor", "gemm"])
@pytest.mark.parametrize("name,M,K,kw", ACT_CASES, ids=[c[0] for c in ACT_CASES])
def test_quant_activations_bit_exact(name, M, K, kw, layout):
    need_gpu()
    x = inputs.activations(M, K, **kw)
    q, s = _gpu_quant(x, layout)
    q_ref, s_ref = _expect(x, layout)
    assert np.array_equal(q, q_ref)
    assert np.array_equal(s, s_ref)
    assert not np.any(s == 0xFF)


def test_quant_weights_bit_exact():
    need_gpu()
    w = inputs.weights(1024, 5120, 0)
    q, s = _gpu_quant(w, 0)
    q_ref, s_ref = _expect(w, 0)
    assert np.array_equal(q, q_ref) and np.array_equal(s, s_ref)


def test_quant_every_bf16_value():
    # Every finite bf16 pattern appears as an element: once in bit order
    # (neighbouring magnitudes share a block) and once shuffled (mixed amax).
    need_gpu()
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = u[(u & 0x7F80) != 0x7F80]
    n = finite.size // 32 * 32
    ordered_blocks = finite[:n].reshape(-1, 32)
    rng = np.random.default_rng(1)
    shuffled = rng.permutation(finite)[:n].reshape(-1, 32)
    for x in (ordered_blocks, shuffled):
        for layout in (0, 1):
            q, s = _gpu_quant(x, layout)
            q_ref, s_ref = _expect(x, layout)
            assert np.array_equal(q, q_ref)
            assert np.array_equal(s, s_ref)


def test_quant_scale_exponent_sweep_with_ties():
    # For every scale byte 0..252, a block whose amax is 2^e (e = byte - 125)
    # and whose other elements sit on the E2M1 rounding midpoints (and one
    # bf16 ulp either side) at that scale; subnormal scales included.
    need_gpu()
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 3.0, 6.0])
    rows = []
    for b in range(0, 253):
        e = b - 125
        unit = 2.0 ** (b - 127)
        vals = np.concatenate([[2.0 ** e], mids * unit])
        lo = F.bf16_to_f64(F.f64_to_bf16(mids * unit) - 1)
        hi = F.bf16_to_f64(F.f64_to_bf16(mids * unit) + 1)
        blk = np.concatenate([vals, lo, hi])[:32]
        blk = np.concatenate([blk, np.zeros(32 - blk.size)])
        blk[1::2] *= -1
        rows.append(blk)
    x = F.f64_to_bf16(np.array(rows))
    for layout in (0, 1):
        q, s = _gpu_quant(x, layout)
        q_ref, s_ref = _expect(x, layout)
        assert np.array_equal(q, q_ref)
        assert np.array_equal(s, s_ref)


def test_quant_strided_input_and_output():
    need_gpu()
    x = inputs.activations(37, 4128, 5, edge=True)
    q, s = _gpu_quant(x, 0, ldx_pad=24, ldq_pad=12)
    q_ref, s_ref = _expect(x, 0)
    assert np.array_equal(q, q_ref) and np.array_equal(s, s_ref)
    q, s = _gpu_quant(x, 1, ldx_pad=24)
    q_ref, s_ref = _expect(x, 1)
    assert np.array_equal(q, q_ref) and np.array_equal(s, s_ref)


@pytest.mark.parametrize("layout,M,K", [(0, 1001, 4128), (1, 1990, 4128)], ids=["rowmajor", "gemm"])
def test_quant_multi_unit_ragged(layout, M, K):
    # Sizes that take the launches handing several row segments (row-major:
    # 9009 of them, not a multiple of the 16 per workgroup; the last segment
    # of every row is one block) or 1 KiB units (GEMM: 4500, the last 16-row
    # strip holding 6 rows) to each wave or workgroup; every byte against
    # the oracle, strided input included.
    need_gpu()
    x = inputs.activations(M, K, 9, outliers=True, edge=True)
    q, s = _gpu_quant(x, layout, ldx_pad=40)
    q_ref, s_ref = _expect(x, layout)
    assert np.array_equal(q, q_ref) and np.array_equal(s, s_ref)


def test_quant_full_prefill_size_sampled_rows():
    # The largest activation of the prefill sweep (8192 x 14336), launched as
    # the GEMM path launches it; the oracle checks sampled rows exactly.
    need_gpu()
    M, K = 8192, 14336
    x = inputs.activations(M, K, 3, outliers=True)
    q, s = _gpu_quant(x, 1)
    rows = np.unique(np.concatenate([[0, 1, M - 1], np.random.default_rng(0).choice(M, 45, replace=False)]))
    q_ref, s_ref = Q.quant_1x32(x[rows])
    rr, kk = np.meshgrid(rows, np.arange(0, K, 2), indexing="ij")
    assert np.array_equal(q[L.weight_byte_offset(0, rr, kk, M, K)], q_ref)
    G = L.gemm_scale_geometry(M, K)[2]
    rr, cc = np.meshgrid(rows, np.arange(K // 32), indexing="ij")
    assert np.array_equal(s[L.gemm_scale_offset(rr, cc, G)], s_ref)


PRESHUFFLE_CASES = [
    ("edge_96x4128", 1, 96, 4128),
    ("linear_1024x5120", 1, 1024, 5120),
    ("kup_16x512x192", 16, 512, 192),
    ("vup_16x256x512", 16, 256, 512),
    ("ragged_3x40x160", 3, 40, 160),
]


def _gpu_preshuffle(w_bits_3d):
    """Row-major GPU quant, then the GPU preshuffle (the checkpoint path)."""
    B, N, K = w_bits_3d.shape
    q, s = mx.mxfp4_quant_1x32(dev_bf16(w_bits_3d.reshape(B * N, K)), mx.MXFP4_LAYOUT_ROWMAJOR)
    d, sc = mx.mxfp4_preshuffle_weight(q, s, N, K, batch=B)
    torch.cuda.synchronize()
    return host_u8(d), host_u8(sc)


@pytest.mark.parametrize("name,B,N,K", PRESHUFFLE_CASES, ids=[c[0] for c in PRESHUFFLE_CASES])
def test_preshuffle_bit_exact(name, B, N, K):
    need_gpu()
    w = np.stack([inputs.weights(N, K, 4, tag=(b,)) for b in range(B)])
    q_ref, s_ref = Q.quant_1x32(w)
    d_ref, sc_ref = L.preshuffle_weight(q_ref, s_ref)
    d, s = _gpu_preshuffle(w)
    assert np.array_equal(d, d_ref)
    assert np.array_equal(s, sc_ref)
    # the load-time helper (direct GEMM-layout quantisation when the batch
    # entries align to 16 rows) produces the same bytes
    W = mx.quantize_weight(dev_bf16(w.reshape(B * N, K)).reshape(B, N, K))
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(W.w_pre), d_ref)
    assert np.array_equal(host_u8(W.ws_pre), sc_ref)


def test_preshuffle_full_size_sampled_strips():
    need_gpu()
    N, K = 34816, 5120
    w = inputs.weights(N, K, 2)
    d, s = _gpu_preshuffle(w[None])
    _, kt, _ = L.weight_geometry(N, K)
    G = L.gemm_scale_geometry(N, K)[2]
    for st in (0, 1, 777, N // 16 - 1):
        q_ref, s_ref = Q.quant_1x32(w[st * 16:(st + 1) * 16])
        d_ref, sc_ref = L.preshuffle_weight(q_ref, s_ref)
        assert np.array_equal(d[st * kt * 1024:(st + 1) * kt * 1024], d_ref)
        assert np.array_equal(s[st * G * 256:(st + 1) * G * 256], sc_ref)
