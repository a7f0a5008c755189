"""Report of the post-cast bar's band reading over the GPU parity checks run
before this module in the same session (pytest collects it last): how often
a bf16 output was more than one ulp from the rounded oracle value -- allowed
only where cancellation makes the pre-cast tolerance band span more than one
bf16 ulp (tests/helpers.check_bf16_cast).  The share must stay small: it is
the tail of near-zero outputs of long sums."""

import pytest

from tests import helpers

pytestmark = pytest.mark.gpu


def test_band_reading_is_rare():
    fr = helpers.BAND_FRACTIONS
    if not fr:
        pytest.skip("no post-cast checks ran in this session")
    worst, mean = max(fr), sum(fr) / len(fr)
    print(f"[band] {len(fr)} checks: mean fraction {mean:.2e}, worst {worst:.2e}")
    assert worst <= 1e-4, worst
