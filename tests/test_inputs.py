"""The seeded input generator: determinism, shapes and the edge-block mix."""

import numpy as np

from mxfp4_block_scaled_quant_amd import inputs
from oracle import formats as F


def test_deterministic_and_shaped():
    a = inputs.linear_problem(16, 64, 256, 0, outliers=True, with_bias=True)
    b = inputs.linear_problem(16, 64, 256, 0, outliers=True, with_bias=True)
    for k in ("x", "w", "bias"):
        assert a[k].dtype == np.uint16 and np.array_equal(a[k], b[k])
    assert a["x"].shape == (16, 256) and a["w"].shape == (64, 256) and a["bias"].shape == (64,)


def test_outlier_channels():
    x = F.bf16_to_f64(inputs.activations(64, 5120, 0, outliers=True))
    col_rms = np.sqrt((x ** 2).mean(axis=0))
    assert (col_rms > 10).sum() == 51          # round(0.01 * 5120)


def test_edge_structure_categories_present():
    x = F.bf16_to_f64(inputs.activations(37, 4128, 5, edge=True)).reshape(37, 129, 32)
    amax = np.abs(x).max(axis=-1)
    zero_blocks = amax == 0
    pow2 = (amax > 0) & (np.frexp(amax)[0] == 0.5)
    assert 0.08 < zero_blocks.mean() < 0.17
    assert pow2.mean() > 0.1
    assert np.any(np.signbit(x) & (x == 0))           # -0.0 present
    assert np.all(np.isfinite(x))
