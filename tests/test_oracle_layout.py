"""Pins of oracle.layout: bijection, fill bytes, hand-placed offsets, an
independent reshape/transpose formulation, and the pages' prior-art order."""

import numpy as np
import pytest

from oracle import layout as L


@pytest.mark.parametrize("rows,K", [(1, 32), (16, 512), (20, 640), (37, 4128),
                                    (300, 256), (64, 5120)])
def test_gemm_scale_layout_bijection_and_fill(rows, K):
    r = np.random.default_rng(rows * 7 + K)
    s = r.integers(0, 255, (rows, K // 32), dtype=np.uint8)   # never 0xFF
    buf = L.scales_to_gemm_layout(s)
    rp, kt, G, nbytes = L.gemm_scale_geometry(rows, K)
    assert buf.size == nbytes == (rp // 16) * G * 256
    assert np.array_equal(L.scales_from_gemm_layout(buf, rows, K), s)
    rr, cc = np.meshgrid(np.arange(rows), np.arange(K // 32), indexing="ij")
    off = L.gemm_scale_offset(rr, cc, G).ravel()
    assert len(np.unique(off)) == off.size and off.max() < nbytes
    mask = np.ones(nbytes, dtype=bool)
    mask[off] = False
    assert np.all(buf[mask] == 0x7F)


def test_gemm_scale_hand_placed_offsets():
    # rows = 20, K = 640: 20 blocks per row, Kt = 5 steps, G = 2 groups,
    # rows padded to 32 -> 2 * 2 * 256 = 1024 bytes.
    rp, kt, G, nbytes = L.gemm_scale_geometry(20, 640)
    assert (rp, kt, G, nbytes) == (32, 5, 2, 1024)
    cases = {(0, 0): 0,          # lane 0, byte 0
             (1, 0): 4,          # next row -> next dword (lane 1)
             (0, 1): 64,         # block kb = 1 -> lane 16
             (0, 4): 1,          # K-step 1 -> byte 1 of the same dword
             (0, 16): 256,       # K-step 4 -> next group tile
             (17, 19): 964}      # row strip 1, group 1, kb 3, row 1: (1*2+1)*256 + 49*4
    for (r, c), off in cases.items():
        assert int(L.gemm_scale_offset(r, c, G)) == off


@pytest.mark.parametrize("rows,K", [(16, 512), (37, 4128), (300, 256)])
def test_gemm_scale_layout_matches_reshape_formulation(rows, K):
    r = np.random.default_rng(5)
    s = r.integers(0, 255, (rows, K // 32), dtype=np.uint8)
    rp, kt, G, nbytes = L.gemm_scale_geometry(rows, K)
    padded = np.full((rp, G * 16), 0x7F, dtype=np.uint8)
    padded[:rows, :K // 32] = s
    # column c = (g*4 + j)*4 + kb; row = rhi*16 + rlo; order (rhi, g, kb, rlo, j)
    alt = padded.reshape(rp // 16, 16, G, 4, 4).transpose(0, 2, 4, 1, 3).ravel()
    assert np.array_equal(L.scales_to_gemm_layout(s), alt)


@pytest.mark.parametrize("B,N,K", [(1, 16, 128), (1, 96, 4128), (2, 40, 192),
                                   (3, 128, 512)])
def test_weight_layout_bijection_and_fill(B, N, K):
    r = np.random.default_rng(B * 1000 + N + K)
    packed = r.integers(0, 256, (B, N, K // 2), dtype=np.uint8)
    sc = r.integers(0, 255, (B, N, K // 32), dtype=np.uint8)
    data, sbuf = L.preshuffle_weight(packed, sc)
    np_, kt, per_b = L.weight_geometry(N, K)
    assert data.size == B * per_b
    p2, s2 = L.unshuffle_weight(data, sbuf, B, N, K)
    assert np.array_equal(p2, packed) and np.array_equal(s2, sc)
    b, n, kk = np.meshgrid(np.arange(B), np.arange(N), np.arange(0, K, 2), indexing="ij")
    off = L.weight_byte_offset(b, n, kk, N, K).ravel()
    assert len(np.unique(off)) == off.size
    mask = np.ones(data.size, dtype=bool)
    mask[off] = False
    assert np.all(data[mask] == 0)


def test_weight_layout_hand_placed_offsets():
    # N = 40 (Np = 48, 3 strips), K = 384 (Kt = 3 steps of 128)
    N, K = 40, 384
    cases = {(0, 0, 0): 0,
             (0, 1, 0): 16,            # next row -> next 16-byte slot (lane 1)
             (0, 0, 2): 1,             # elements 2,3 -> next byte
             (0, 0, 32): 256,          # block kb = 1 -> slot 16
             (0, 0, 128): 1024,        # K-step 1 -> next 1 KiB unit
             (0, 17, 130): (1 * 3 + 1) * 1024 + 1 * 16 + 1,   # strip 1, step 1, row 1
             (1, 0, 0): 3 * 3 * 1024}              # next batch entry
    for (b, n, k), off in cases.items():
        assert int(L.weight_byte_offset(b, n, k, N, K)) == off


@pytest.mark.parametrize("N,K", [(16, 128), (40, 4128)])
def test_weight_layout_matches_reshape_formulation(N, K):
    r = np.random.default_rng(9)
    packed = r.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sc = r.integers(0, 255, (N, K // 32), dtype=np.uint8)
    np_, kt, per_b = L.weight_geometry(N, K)
    padded = np.zeros((np_, kt * 64), dtype=np.uint8)
    padded[:N, :K // 2] = packed
    # byte column = t*64 + kb*16 + e2; row = s*16 + r; order (s, t, kb, r, e2)
    alt = padded.reshape(np_ // 16, 16, kt, 4, 16).transpose(0, 2, 3, 1, 4).ravel()
    data, _ = L.preshuffle_weight(packed, sc)
    assert np.array_equal(data, alt)


@pytest.mark.parametrize("rows,cols", [(32, 8), (64, 24)])
def test_prior_art_order_matches_pages_axis_order(rows, cols):
    # P2 §2 describes the prior-art swizzle as a split of the row index into
    # (32-row tile, 16-row half, row in half) and of the column index into
    # (8-column tile, 4-column half, column in half), emitted in the order
    # row tile, column tile, column in half, row in half, column half, row
    # half; P2 §3 checks it on a counting input.  Enumerate that order with a
    # loop nest and compare with the closed-form offsets.
    src = np.arange(rows * cols).reshape(rows, cols)
    emitted = []
    for rt in range(rows // 32):
        for ct in range(cols // 8):
            for cl in range(4):
                for rl in range(16):
                    for ch in range(2):
                        for rh in range(2):
                            emitted.append(src[rt * 32 + rh * 16 + rl, ct * 8 + ch * 4 + cl])
    emitted = np.array(emitted)
    r, c = np.meshgrid(np.arange(rows), np.arange(cols), indexing="ij")
    off = L.prior_art_scale_offset(r, c, cols)
    assert np.array_equal(emitted[off], src)
