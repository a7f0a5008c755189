"""Scale and weight layouts as explicit index maps (CPU oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

The pages load weights once, preshuffle them into the layout the FP4 GEMM
reads, and swizzle the E8M0 scales into a tile order, padding scale tiles
with E8M0 1.0 (0x7F) and never with 0xFF, which is NaN (P1 §Modifications;
P2 §2, the scale swizzle and activation-scale padding helpers).  The
prior-art tile order is printed there; the weight permutation is not.  This
library uses its own layouts, defined here as index maps and nothing else:

GEMM scale layout (activation scales and weight scales alike)
    R rows, C = K/32 blocks per row, Kt = ceil(K/128) K-steps,
    G = ceil(Kt/4) step groups, Rp = 16*ceil(R/16).
    Scale (r, c): t = c // 4, kb = c % 4, g = t // 4, j = t % 4,
        byte = ((r // 16) * G + g) * 256 + (kb * 16 + r % 16) * 4 + j.
    One 256-byte tile holds 16 rows x 16 blocks (512 K).  Its dword number
    kb*16 + r%16 is the lane of a 16x16x128 block-scaled MFMA that consumes
    row r's block kb, and byte j selects the K-step within the group.
    Size Rp/16 * G * 256 bytes; every byte that is not a real scale is 0x7F.

Preshuffled weight layout (W4A4 GEMM and A16WFP4 BMM weights)
    per batch entry, N rows, K; Np = 16*ceil(N/16), Kt = ceil(K/128).
    The byte holding elements (n, k) and (n, k+1), k even:
        s = n // 16, r = n % 16, t = k // 128, kb = (k % 128) // 32, e = k % 32,
        byte = ((b * Np/16 + s) * Kt + t) * 1024 + (kb * 16 + r) * 16 + e // 2,
    element k in the low nibble.  One 1 KiB unit is a 16-row x 128-K tile;
    its 16-byte slot kb*16 + r is one whole 1x32 block, the operand of MFMA
    lane kb*16 + r.  Units of one 16-row strip run contiguously along K.
    Size B * Np/16 * Kt * 1024 bytes; padding bytes are 0x00 (FP4 +0).
    Weight scales for it use the GEMM scale layout per batch entry, with the
    batch entries concatenated.

GEMM activation layout
    Quantised activations for the GEMM use the preshuffled weight layout
    with the M rows in place of N (batch 1): 1 KiB units of 16 rows x 128 K,
    slot kb*16 + r = row r's block kb, rows padded to 16 and K to 128 with
    zero bytes; their scales use the GEMM scale layout.  So a weight prepared
    by quantising straight into the GEMM layout is bytewise the preshuffled
    weight.

Pins (tests/test_oracle_layout.py): forward/inverse bijection over all
in-range indices; every non-image byte is the documented fill; hand-placed
positions worked from the formulas above; an independent reshape/transpose
formulation of each map; the prior-art order decoded from the pages'
printed 32x8 reshape/permute, checked on an arange input as P2 §3's unit
test does.
"""

from __future__ import annotations

import numpy as np

from .formats import E8M0_ONE


def _cdiv(a, b):
    return -(-a // b)


# --------------------------------------------------------------------------
# GEMM scale layout
# --------------------------------------------------------------------------

def gemm_scale_geometry(rows: int, K: int):
    """(Rp, Kt, G, nbytes) of the GEMM scale layout for rows x K."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    rp = 16 * _cdiv(rows, 16)
    kt = _cdiv(K, 128)
    g = _cdiv(kt, 4)
    return rp, kt, g, (rp // 16) * g * 256


def gemm_scale_offset(r, c, G):
    """Byte offset of scale (r, c) in the GEMM scale layout with G groups."""
    r = np.asarray(r, dtype=np.int64)
    c = np.asarray(c, dtype=np.int64)
    t, kb = c // 4, c % 4
    g, j = t // 4, t % 4
    return ((r // 16) * G + g) * 256 + (kb * 16 + r % 16) * 4 + j


def scales_to_gemm_layout(scales_rm):
    """Row-major scales [R, K/32] (uint8) -> GEMM-layout bytes (uint8, 1-D)."""
    scales_rm = np.asarray(scales_rm, dtype=np.uint8)
    rows, cols = scales_rm.shape
    _, _, G, nbytes = gemm_scale_geometry(rows, cols * 32)
    out = np.full(nbytes, E8M0_ONE, dtype=np.uint8)
    r, c = np.meshgrid(np.arange(rows), np.arange(cols), indexing="ij")
    out[gemm_scale_offset(r, c, G)] = scales_rm
    return out


def scales_from_gemm_layout(buf, rows: int, K: int):
    """Inverse of :func:`scales_to_gemm_layout` (reads the real scales only)."""
    _, _, G, nbytes = gemm_scale_geometry(rows, K)
    buf = np.asarray(buf, dtype=np.uint8)
    if buf.size != nbytes:
        raise ValueError("buffer size does not match the layout")
    r, c = np.meshgrid(np.arange(rows), np.arange(K // 32), indexing="ij")
    return buf[gemm_scale_offset(r, c, G)]


# --------------------------------------------------------------------------
# Preshuffled weight layout
# --------------------------------------------------------------------------

def weight_geometry(N: int, K: int):
    """(Np, Kt, data bytes per batch entry) of the preshuffled weight layout."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    np_ = 16 * _cdiv(N, 16)
    kt = _cdiv(K, 128)
    return np_, kt, (np_ // 16) * kt * 1024


def weight_byte_offset(b, n, k, N, K):
    """Byte offset of the pair (n, k), (n, k+1) (k even) for batch entry b."""
    np_, kt, _ = weight_geometry(N, K)
    b = np.asarray(b, dtype=np.int64)
    n = np.asarray(n, dtype=np.int64)
    k = np.asarray(k, dtype=np.int64)
    s, r = n // 16, n % 16
    t, kb, e = k // 128, (k % 128) // 32, k % 32
    return ((b * (np_ // 16) + s) * kt + t) * 1024 + (kb * 16 + r) * 16 + e // 2


def preshuffle_weight(packed, scales_rm):
    """Packed FP4 [B, N, K/2] + row-major scales [B, N, K/32] -> (data, scales).

    A 2-D input (one matrix) is treated as B = 1.  Returns two 1-D uint8
    arrays: the preshuffled data (zero padded) and the concatenated per-batch
    GEMM-layout scales (0x7F padded).
    """
    packed = np.asarray(packed, dtype=np.uint8)
    scales_rm = np.asarray(scales_rm, dtype=np.uint8)
    if packed.ndim == 2:
        packed, scales_rm = packed[None], scales_rm[None]
    B, N, half_k = packed.shape
    K = half_k * 2
    if scales_rm.shape != (B, N, K // 32):
        raise ValueError("scale shape does not match the data")
    _, _, per_b = weight_geometry(N, K)
    data = np.zeros(B * per_b, dtype=np.uint8)
    b, n, kk = np.meshgrid(np.arange(B), np.arange(N), np.arange(0, K, 2),
                           indexing="ij")
    data[weight_byte_offset(b, n, kk, N, K)] = packed
    sc = np.concatenate([scales_to_gemm_layout(scales_rm[i]) for i in range(B)])
    return data, sc


def unshuffle_weight(data, scales, B: int, N: int, K: int):
    """Inverse of :func:`preshuffle_weight`: -> (packed [B,N,K/2], scales [B,N,K/32])."""
    _, _, per_b = weight_geometry(N, K)
    data = np.asarray(data, dtype=np.uint8)
    if data.size != B * per_b:
        raise ValueError("data size does not match the layout")
    b, n, kk = np.meshgrid(np.arange(B), np.arange(N), np.arange(0, K, 2),
                           indexing="ij")
    packed = data[weight_byte_offset(b, n, kk, N, K)]
    sbytes = gemm_scale_geometry(N, K)[3]
    scales = np.asarray(scales, dtype=np.uint8).reshape(B, sbytes)
    sc = np.stack([scales_from_gemm_layout(scales[i], N, K) for i in range(B)])
    return packed, sc


def to_gemm_layout(packed, scales_rm):
    """Row-major packed FP4 [R, K/2] + scales [R, K/32] -> GEMM-layout (data, scales).

    The activation form of the preshuffled layout (batch 1)."""
    return preshuffle_weight(np.asarray(packed)[None], np.asarray(scales_rm)[None])


# --------------------------------------------------------------------------
# The pages' prior-art scale tile order (context; not used by this library)
# --------------------------------------------------------------------------

def prior_art_scale_offset(r, c, cols):
    """Element offset of scale (r, c) in the pages' 32x8-tile swizzle.

    Decoded from the reshape/permute printed in P2 §2 (the scale swizzle
    helper): rows split as (r//32, (r%32)//16, r%16), columns as
    (c//8, (c%8)//4, c%4), reordered to (r//32, c//8, c%4, r%16, (c%8)//4,
    (r%32)//16).  So each 256-entry tile is a 32-row x 8-column block; inside
    it the dword index is (c%4)*16 + r%16 and the byte inside the dword is
    ((c%8)//4)*2 + (r%32)//16.
    """
    r = np.asarray(r, dtype=np.int64)
    c = np.asarray(c, dtype=np.int64)
    tile = (r // 32) * (cols // 8) + c // 8
    dword = (c % 4) * 16 + r % 16
    byte = ((c % 8) // 4) * 2 + (r % 32) // 16
    return tile * 256 + dword * 4 + byte
