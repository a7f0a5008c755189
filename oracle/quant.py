"""Per-1x32 MXFP4 quantisation and dequantisation (CPU oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

What is computed.  P1 §Modifications and P2 §2 (``apply_weights`` and the
registered quantisation op) quantise bf16 activations per 1x32 block along K
into packed FP4 (two codes per byte, ``[rows, K/2]``) plus one E8M0 scale per
block (``[rows, K/32]``); weights are stored the same way.  The pages do not
spell out the arithmetic, so this follows the OCP-MX conversion of a vector
of scalars into one MX block, with the readings below:

1. amax = max |v_i| over the 32 values (exact).
2. shared exponent = floor(log2(amax)) - emax(E2M1) with emax = 2, computed
   exactly from the binary exponent (frexp), never with a floating log2;
   clamped to the E8M0 range, so the scale byte is
   b = clamp(floor(log2 amax) - 2 + 127, 0, 254).  An all-zero block or a
   subnormal amax gives b = 0; the largest bf16 gives 252; 0xFF (NaN) is
   never produced.
3. y_i = v_i / 2^(b-127) (exact: a power-of-two scaling of a bf16 value).
4. |y_i| goes to the nearest E2M1 magnitude; a tie goes to the code whose
   lowest bit is 0 (round-to-nearest-even); |y_i| > 6 saturates to 6 (the
   nearest-magnitude search over the finite table yields this by itself).
5. the sign bit is the sign bit of v_i (so -0.0 and tiny negatives that round
   to zero encode as 0x8).
6. element 2j goes to the low nibble of byte j, element 2j+1 to the high
   nibble (the ``float4_e2m1fn_x2`` packing named in P2 §2).

Step 4 is a brute-force nearest search with an explicit tie rule, written to
be checked by eye, not a bit trick.

Pins (tests/test_oracle_quant.py): exhaustive scale rule over every finite
positive bf16 amax; element rounding against an independent
``fractions.Fraction`` nearest-even implementation over every bf16 value in
several binades; hand-worked blocks (tests/golden/worked_blocks.json);
idempotence Q(dq(Q(x))) == Q(x); power-of-two equivariance; sign symmetry.
"""

from __future__ import annotations

import numpy as np

from .formats import E2M1_EMAX, E2M1_MAGNITUDES, E2M1_TABLE, bf16_to_f64

BLOCK = 32


def scale_byte(amax):
    """E8M0 scale byte for block amax values (fp64, >= 0), step 2 above."""
    amax = np.asarray(amax, dtype=np.float64)
    if np.any(amax < 0) or not np.all(np.isfinite(amax)):
        raise ValueError("scale_byte: amax must be finite and >= 0")
    _, e = np.frexp(amax)          # amax = f * 2^e with f in [0.5, 1)
    floor_log2 = e - 1
    b = np.clip(floor_log2 - E2M1_EMAX + 127, 0, 254)
    return np.where(amax == 0, 0, b).astype(np.uint8)


def round_to_e2m1_magnitude(y):
    """Index (0..7) of the nearest E2M1 magnitude to y >= 0, ties to even.

    Brute force: distance to each of the 8 magnitudes (exact in fp64 for the
    dyadic inputs that occur), keep the smallest; among equal distances keep
    the even code.  Values above 6 land on code 7 (6.0): saturation.
    """
    y = np.asarray(y, dtype=np.float64)
    if np.any(y < 0):
        raise ValueError("magnitude must be >= 0")
    d = np.abs(y[..., None] - E2M1_MAGNITUDES)          # [..., 8]
    dmin = d.min(axis=-1, keepdims=True)
    is_min = d == dmin
    even = (np.arange(8) % 2) == 0
    # Prefer an even code among the minima; otherwise the (single) odd one.
    pick_even = is_min & even
    has_even = pick_even.any(axis=-1)
    idx_even = np.argmax(pick_even, axis=-1)
    idx_any = np.argmax(is_min, axis=-1)
    return np.where(has_even, idx_even, idx_any).astype(np.uint8)


def quant_blocks_f64(v):
    """Quantise fp64 values shaped [..., nblocks, 32] (each exactly a bf16 value).

    Returns (codes uint8 [..., nblocks, 32] in 0..15, scale bytes uint8
    [..., nblocks]).
    """
    v = np.asarray(v, dtype=np.float64)
    if v.shape[-1] != BLOCK:
        raise ValueError("last axis must be one 1x32 block")
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite input is outside the contract")
    amax = np.abs(v).max(axis=-1)
    b = scale_byte(amax)
    y = np.ldexp(np.abs(v), 127 - b[..., None].astype(np.int64))
    mag = round_to_e2m1_magnitude(y)
    sign = np.signbit(v).astype(np.uint8)
    codes = (sign << 3) | mag
    return codes, b


def pack_codes(codes):
    """Pack codes [..., K] (K even) into bytes [..., K/2], low nibble first."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed):
    """Inverse of :func:`pack_codes`: bytes [..., K/2] -> codes [..., K]."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def quant_1x32(x_bf16_bits):
    """bf16 bit patterns [..., rows, K] (K % 32 == 0) -> (packed FP4, scales).

    packed: uint8 [..., rows, K/2]; scales: uint8 [..., rows, K/32] row-major
    (the unpadded forms named in P2 §2 for the quantisation op's outputs).
    """
    x = bf16_to_f64(x_bf16_bits)
    *lead, rows, k = x.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = x.reshape(*lead, rows, k // BLOCK, BLOCK)
    codes, b = quant_blocks_f64(blocks)
    return pack_codes(codes.reshape(*lead, rows, k)), b


def dequant(packed, scales):
    """Packed FP4 [..., rows, K/2] + scales [..., rows, K/32] -> fp64 [..., rows, K].

    dq = E2M1 value * 2^(b - 127), exact in fp64.
    """
    codes = unpack_codes(packed)
    vals = E2M1_TABLE[codes]
    *lead, rows, k = vals.shape
    scales = np.asarray(scales, dtype=np.int64)
    if scales.shape != tuple(lead) + (rows, k // BLOCK):
        raise ValueError("scale shape does not match packed data")
    blocks = vals.reshape(*lead, rows, k // BLOCK, BLOCK)
    blocks = np.ldexp(blocks, (scales - 127)[..., None])
    # 0xFF is NaN in E8M0: a block scaled by it is NaN whatever its codes.
    blocks = np.where((scales == 0xFF)[..., None], np.nan, blocks)
    return blocks.reshape(*lead, rows, k)
