"""Element and scale formats: E2M1 (FP4), E8M0 (block scale) and bf16.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

Every function here is the closed-form definition from OCP-MX (E2M1, E8M0)
or IEEE-754-style binary formats (bf16), written out directly.  P1 §Modifications
and P2 §2 (the scheme diff) name the formats -- packed FP4 viewed as
``float4_e2m1fn_x2`` and E8M0 scales viewed as ``float8_e8m0fnu``, with 0xFF
being NaN -- but do not define them.

Pins (tests/test_oracle_formats.py):
  * E2M1 table: the 16 closed-form values against the magnitudes listed by
    OCP-MX for E2M1 (0, 0.5, 1, 1.5, 2, 3, 4, 6) and sign symmetry.
  * E8M0: 2^(b-127) against torch's float8_e8m0fnu cast, 0xFF is NaN.
  * bf16 decode: against torch's bfloat16 -> float32 cast for all 65536
    patterns.
  * fp64 -> bf16 RNE: against an integer bit-rounding reference on fp32
    inputs (exhaustive over a wide band of fp32 patterns), torch's
    float32 -> bfloat16 cast, and hand-placed ties, overflow and subnormals.
"""

from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no Inf / NaN.
# --------------------------------------------------------------------------

E2M1_EMAX = 2
"""Exponent of the largest E2M1 normal number (6 = 1.5 * 2^2), OCP-MX."""

E2M1_MAX = 6.0


def e2m1_value(code: int) -> float:
    """Value of one 4-bit E2M1 code (OCP-MX element format E2M1).

    code = s*8 + e*2 + m.  e == 0 is subnormal: (-1)^s * 0.5 * m.
    e > 0 is normal: (-1)^s * 2^(e-1) * (1 + m/2).
    """
    if not 0 <= code <= 15:
        raise ValueError("E2M1 code out of range")
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = 0.5 * m
    else:
        mag = 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -mag if s else mag


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
"""Decoded value of every code 0..15 (code 8 is -0.0)."""

E2M1_MAGNITUDES = E2M1_TABLE[:8].copy()
"""Magnitudes of codes 0..7, increasing."""


# --------------------------------------------------------------------------
# E8M0: 8 exponent bits, bias 127, no sign, no mantissa; 0xFF is NaN.
# --------------------------------------------------------------------------

E8M0_BIAS = 127
E8M0_ONE = 0x7F
"""E8M0 encoding of 1.0; the fill value for padded scales (P2 §2, the
activation-scale padding helper: pad with 1.0, since 0xFF is NaN)."""
E8M0_NAN = 0xFF


def e8m0_value(b):
    """Decode E8M0 bytes to fp64: 2^(b - 127), NaN for 0xFF (OCP-MX)."""
    b = np.asarray(b, dtype=np.int64)
    out = np.ldexp(1.0, b - E8M0_BIAS).astype(np.float64)
    return np.where(b == E8M0_NAN, np.nan, out)


# --------------------------------------------------------------------------
# bf16: the top 16 bits of an IEEE binary32.
# --------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as fp64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round fp64 values to bf16 with round-to-nearest-even; return uint16 bits.

    Done in one rounding from fp64 (never through fp32, which could round
    twice): split |x| = f * 2^e with f in [0.5, 1), round to the bf16 quantum
    2^(e-8) (8 significant bits), or 2^-133 below the normal range, with
    numpy's rint (ties to even), and map results of magnitude 2^128 or more
    to infinity.  The rounded value is exactly representable in fp32, so the
    final fp32 view is exact.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("f64_to_bf16: non-finite input")
    _, e = np.frexp(x)
    q_exp = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(x, -q_exp)), q_exp)
    with np.errstate(over="ignore"):
        big = np.abs(r) >= 2.0 ** 128
        r32 = np.where(big, np.copysign(np.inf, x), r).astype(np.float32)
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    # rint(-tiny) gives -0.0, which keeps the sign bit as IEEE rounding does.
    return bits


def f32_to_bf16_bits_reference(u32) -> np.ndarray:
    """Integer round-to-nearest-even of fp32 bit patterns to bf16 bits.

    An independent formulation used only to pin :func:`f64_to_bf16`: add
    0x7FFF plus the lowest kept bit, then truncate the low 16 bits.  Valid for
    finite inputs (overflow carries into the exponent and yields Inf).
    """
    u = np.asarray(u32, dtype=np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
