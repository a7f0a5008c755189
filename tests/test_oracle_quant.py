"""Pins of oracle.quant: scale rule, element rounding, worked blocks, invariants."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import quant as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_blocks.json")


def _bf16_bits_of(values):
    x = np.array(values, dtype=np.float64)
    bits = F.f64_to_bf16(x)
    assert np.array_equal(F.bf16_to_f64(bits), x), "fixture value is not a bf16 number"
    return bits


def _all_finite_positive_bf16():
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint32).astype(np.uint16)
    return bits, F.bf16_to_f64(bits)


def test_scale_rule_exhaustive_over_bf16_amax():
    _, amax = _all_finite_positive_bf16()
    b = Q.scale_byte(amax).astype(np.int64)
    assert b.max() == 252 and b.min() == 0
    ratio = amax / np.ldexp(1.0, b - 127)
    normal = amax >= 2.0 ** -125          # biased exponent field E >= 2
    assert np.all((ratio[normal] >= 4) & (ratio[normal] < 8))
    assert np.all(b[~normal] == 0)
    assert np.all(ratio[~normal] < 4)
    pow2 = normal & (np.frexp(amax)[0] == 0.5)
    assert np.all(ratio[pow2] == 4.0)
    assert Q.scale_byte(0.0) == 0


def test_scale_rule_golden():
    with open(GOLDEN) as f:
        g = json.load(f)
    for case in g["scale_rule"]:
        amax = float.fromhex(case["amax"])
        assert int(Q.scale_byte(amax)) == case["b"], case


def _fraction_nearest_even(y: Fraction) -> int:
    """Independent reference: walk the E2M1 magnitude intervals in exact
    rationals; below a midpoint go down, above go up, on it pick the even
    code; at or above 6 saturate to code 7."""
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
            Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
    if y >= mags[-1]:
        return 7
    for i in range(7):
        lo, hi = mags[i], mags[i + 1]
        if lo <= y <= hi:
            mid = (lo + hi) / 2
            if y < mid:
                return i
            if y > mid:
                return i + 1
            return i if i % 2 == 0 else i + 1
    raise AssertionError("unreachable")


def test_element_rounding_matches_fraction_reference():
    # Every non-negative bf16 value in [2^-12, 16): all scaled magnitudes that
    # can reach step 4 (amax scales into [4, 8)), plus the saturating range.
    _, vals = _all_finite_positive_bf16()
    y = vals[(vals >= 2.0 ** -12) & (vals < 16.0)]
    y = np.concatenate([[0.0], y])
    ours = Q.round_to_e2m1_magnitude(y)
    ref = np.array([_fraction_nearest_even(Fraction(float(v))) for v in y])
    assert np.array_equal(ours, ref)


def test_midpoints_and_neighbours():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    expect_code = [0, 2, 2, 4, 4, 6, 6]    # ties to the even code
    for m, c in zip(mids, expect_code):
        assert Q.round_to_e2m1_magnitude(np.array([m]))[0] == c
        # one bf16 ulp either side leaves the tie
        up = np.nextafter(np.float32(m), np.float32(np.inf))
        lo_bits = F.f64_to_bf16(np.array([m])) - 1
        hi_bits = F.f64_to_bf16(np.array([m])) + 1
        lo_v = F.bf16_to_f64(lo_bits)[0]
        hi_v = F.bf16_to_f64(hi_bits)[0]
        assert Q.round_to_e2m1_magnitude(np.array([lo_v]))[0] == \
            _fraction_nearest_even(Fraction(lo_v))
        assert Q.round_to_e2m1_magnitude(np.array([hi_v]))[0] == \
            _fraction_nearest_even(Fraction(hi_v))
        assert up > m


def test_worked_blocks():
    with open(GOLDEN) as f:
        g = json.load(f)
    for blk in g["blocks"]:
        vals = [float.fromhex(v) for v in blk["values"]]
        vals = vals + [0.0] * (32 - len(vals))
        bits = _bf16_bits_of(vals)[None, :]
        packed, scales = Q.quant_1x32(bits)
        assert int(scales[0, 0]) == blk["scale"], blk["name"]
        codes = Q.unpack_codes(packed)[0]
        n = len(blk["codes"])
        assert list(codes[:n]) == blk["codes"], blk["name"]
        assert np.all(codes[n:] == 0), blk["name"]
        nb = len(blk["packed_first_bytes"])
        assert list(packed[0, :nb]) == blk["packed_first_bytes"], blk["name"]


def _random_blocks(seed, nblocks, spread=8):
    r = np.random.default_rng(seed)
    v = r.standard_normal((nblocks, 32)) * np.ldexp(1.0, r.integers(-spread, spread, (nblocks, 1)))
    return F.f64_to_bf16(v)


def test_idempotence():
    bits = _random_blocks(1, 4000, spread=40)
    packed, scales = Q.quant_1x32(bits)
    dq = Q.dequant(packed, scales)
    dq_bits = F.f64_to_bf16(dq)
    assert np.array_equal(F.bf16_to_f64(dq_bits), dq)     # dq is exactly bf16
    p2, s2 = Q.quant_1x32(dq_bits)
    assert np.array_equal(p2, packed) and np.array_equal(s2, scales)


@pytest.mark.parametrize("j", [-9, -1, 1, 5, 17])
def test_power_of_two_equivariance(j):
    bits = _random_blocks(2, 2000, spread=6)
    x = F.bf16_to_f64(bits)
    xs = np.ldexp(x, j)
    xs_bits = F.f64_to_bf16(xs)
    assert np.array_equal(F.bf16_to_f64(xs_bits), xs)
    p0, s0 = Q.quant_1x32(bits)
    p1, s1 = Q.quant_1x32(xs_bits)
    assert np.array_equal(p0, p1)
    assert np.array_equal(s1.astype(int), s0.astype(int) + j)


def test_sign_symmetry():
    bits = _random_blocks(3, 2000)
    p0, s0 = Q.quant_1x32(bits)
    p1, s1 = Q.quant_1x32(bits ^ np.uint16(0x8000))
    assert np.array_equal(s0, s1)
    assert np.array_equal(Q.unpack_codes(p1), Q.unpack_codes(p0) ^ 8)


def test_quantisation_error_bound():
    # Within the non-saturating range the error is at most half a step of
    # the E2M1 grid at the block scale: <= 2^(b-127) (step 2 near 4..6) / 2.
    bits = _random_blocks(4, 3000)
    x = F.bf16_to_f64(bits).reshape(-1, 32)
    packed, scales = Q.quant_1x32(bits)
    dq = Q.dequant(packed, scales).reshape(-1, 32)
    unit = np.ldexp(1.0, scales.reshape(-1, 1).astype(int) - 127)
    y = np.abs(x) / unit
    err = np.abs(dq - x) / unit
    inside = y <= 6
    assert np.all(err[inside] <= 1.0)
    assert np.all(err[~inside] <= 2.0)     # saturation: y in (6, 8)
    assert np.all(np.sign(dq[dq != 0]) == np.sign(x[dq != 0]))


def test_packing_roundtrip_and_order():
    codes = np.arange(32, dtype=np.uint8)[None, :] % 16
    p = Q.pack_codes(codes)
    assert p[0, 0] == (0 | (1 << 4)) and p[0, 1] == (2 | (3 << 4))
    assert np.array_equal(Q.unpack_codes(p), codes)


def test_dequant_of_nan_scale_is_nan():
    p = np.zeros((1, 16), dtype=np.uint8)
    assert np.all(np.isnan(Q.dequant(p, np.array([[0xFF]], dtype=np.uint8))))
    assert np.all(Q.dequant(p, np.array([[0x7F]], dtype=np.uint8)) == 0)


def test_rejects_bad_shapes_and_nonfinite():
    with pytest.raises(ValueError):
        Q.quant_1x32(np.zeros((1, 48), dtype=np.uint16))
    with pytest.raises(ValueError):
        Q.quant_1x32(np.full((1, 32), 0x7F80, dtype=np.uint16))   # +Inf
