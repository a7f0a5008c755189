"""Pins of oracle.formats against things other than itself (CPU only)."""

import numpy as np
import pytest
import torch

from oracle import formats as F


def test_e2m1_table_matches_ocp_magnitudes():
    # OCP-MX lists the E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
    assert list(F.E2M1_MAGNITUDES) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    # Codes 8..15 are the negatives (sign bit 3), code 8 is -0.0.
    assert np.array_equal(F.E2M1_TABLE[8:], -F.E2M1_TABLE[:8])
    assert np.signbit(F.E2M1_TABLE[8]) and not np.signbit(F.E2M1_TABLE[0])
    assert F.E2M1_MAX == F.E2M1_TABLE.max() == 1.5 * 2.0 ** F.E2M1_EMAX


def test_e8m0_decode_against_torch():
    b = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(F.e8m0_value(b), ref)
    assert F.e8m0_value(F.E8M0_ONE) == 1.0
    assert np.isnan(F.e8m0_value(0xFF))
    # torch also decodes 0xFF as NaN.
    t = torch.tensor([0xFF], dtype=torch.uint8).view(torch.float8_e8m0fnu).float()
    assert torch.isnan(t).all()


def test_bf16_decode_all_patterns_against_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = F.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert np.array_equal(np.signbit(ours[~both_nan]), np.signbit(ref[~both_nan]))


def _finite_f32_band(lo_exp, hi_exp, step):
    """fp32 bit patterns with biased exponent in [lo_exp, hi_exp], both signs."""
    u = np.arange(lo_exp << 23, (hi_exp + 1) << 23, step, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([u, u | np.uint32(0x80000000)])


@pytest.mark.parametrize("lo,hi,step", [(0, 2, 1), (100, 101, 1), (120, 134, 7),
                                         (250, 254, 3)])
def test_f64_to_bf16_matches_integer_rounding(lo, hi, step):
    u = _finite_f32_band(lo, hi, step)
    x = u.view(np.float32).astype(np.float64)
    ours = F.f64_to_bf16(x)
    ref = F.f32_to_bf16_bits_reference(u)
    assert np.array_equal(ours, ref)


def test_f64_to_bf16_matches_torch_cast():
    r = np.random.default_rng(7)
    x = np.concatenate([r.standard_normal(200000) * 10.0 ** r.integers(-30, 30, 200000),
                        np.ldexp(r.random(1000), -140)]).astype(np.float32)
    ours = F.f64_to_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f64_to_bf16_rounds_once_from_fp64():
    # 1 + 2^-8 + 2^-30 is just above the bf16 midpoint 1 + 2^-8: correct RNE
    # from fp64 rounds up to 1 + 2^-7.  Rounding to fp32 first would give
    # 1 + 2^-8 exactly (the 2^-30 is lost) and then a tie to even -> 1.0.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert F.bf16_to_f64(F.f64_to_bf16(np.array([x])))[0] == 1.0 + 2.0 ** -7
    # Exact ties go to even.
    assert F.bf16_to_f64(F.f64_to_bf16(np.array([1.0 + 2.0 ** -8])))[0] == 1.0
    assert F.bf16_to_f64(F.f64_to_bf16(np.array([1.0 + 3 * 2.0 ** -8])))[0] == 1.0 + 2.0 ** -6
    # Signed zero, overflow to Inf, smallest subnormal.
    assert F.f64_to_bf16(np.array([-0.0]))[0] == 0x8000
    assert F.f64_to_bf16(np.array([3.5e38]))[0] == 0x7F80
    assert F.f64_to_bf16(np.array([2.0 ** -133]))[0] == 0x0001
    assert F.f64_to_bf16(np.array([2.0 ** -134]))[0] == 0x0000      # tie -> even (0)
    assert F.f64_to_bf16(np.array([1.5 * 2.0 ** -133]))[0] == 0x0002  # tie -> even (2)
