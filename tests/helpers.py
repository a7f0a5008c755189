"""Shared helpers for the parity tests (conversion, comparison, sampling)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

TOL_REL = 2.0 ** -18     # |y_gpu - y_ref| <= 2^-18 * (sum |a_i b_i| + |bias|) before the cast


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint8)


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def ordered(bits: np.ndarray) -> np.ndarray:
    """Map bf16 bit patterns to integers whose order is the numeric order."""
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    return np.abs(ordered(a_bits) - ordered(b_bits))


def check_f32_tolerance(y_gpu: np.ndarray, y_ref: np.ndarray, abs_sum: np.ndarray,
                        bias_abs: np.ndarray | None = None) -> float:
    """Assert the pre-cast bar; return the worst ratio err / bound (<= 1)."""
    assert np.all(np.isfinite(y_gpu)), "non-finite output"
    bound = TOL_REL * (abs_sum + (0.0 if bias_abs is None else bias_abs))
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= 1.0, f"tolerance exceeded: worst err/bound = {worst:.3g}"
    return worst


def tolerance_bound(abs_sum: np.ndarray, bias_abs: np.ndarray | None = None) -> np.ndarray:
    return TOL_REL * (abs_sum + (0.0 if bias_abs is None else bias_abs))


def check_bf16_cast(y_bits: np.ndarray, y_ref: np.ndarray, bound: np.ndarray) -> float:
    """Post-cast bar: each bf16 output is within 1 ulp of RNE(y_ref), or, where
    the pre-cast tolerance band is wider than that (cancellation: |y| much
    smaller than sum |a_i b_i|), it is the RNE of some value inside the band,
    i.e. between RNE(y_ref - bound) and RNE(y_ref + bound) (RNE is monotone).
    Returns the fraction of elements that needed the band reading."""
    from oracle.linalg import to_bf16
    ref_bits = to_bf16(y_ref)
    within_ulp = ulp_distance(y_bits, ref_bits) <= 1
    lo = ordered(to_bf16(y_ref - bound))
    hi = ordered(to_bf16(y_ref + bound))
    o = ordered(y_bits)
    in_band = (o >= lo) & (o <= hi)
    # the band reading only where the strict bar is out of reach: the rounded
    # band spans more than one bf16 ulp there
    wide = (hi - lo) >= 2
    bad = ~(within_ulp | (in_band & wide))
    assert not bad.any(), (f"{int(bad.sum())} bf16 outputs neither within 1 ulp nor inside "
                           f"a rounded tolerance band wider than 1 ulp; worst ulp distance "
                           f"{int(ulp_distance(y_bits, ref_bits)[bad].max())}")
    frac = float((~within_ulp).mean()) if y_bits.size else 0.0
    BAND_FRACTIONS.append(frac)
    return frac


# fraction of outputs that needed the band reading, one entry per check
# (reported by tests/test_zz_band_report.py)
BAND_FRACTIONS: list = []
