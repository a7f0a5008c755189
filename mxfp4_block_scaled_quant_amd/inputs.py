"""Seeded synthetic inputs shared by the tests, the bench and the CPU oracle.

This module holds no arithmetic of the method (no quantisation, scaling,
rounding to FP4 or GEMM).  It draws fp32 samples with numpy, shapes them into
the structure of each workload, and converts them to bf16 with torch's
float32 -> bfloat16 cast (round-to-nearest-even, a library routine).  Both
the HIP path and the oracle consume the same returned bf16 bit patterns.

Every stream is ``numpy.random.default_rng([seed, role, *dims])`` with role
0 = activations, 1 = weights, 2 = bias, 3 = outlier channels, 4 = edge-block
structure, so each tensor is reproducible on its own.

Workloads (shapes from P1 §Accuracy Tests -- the (16, 1024, 5120) check --
and from the hidden sizes the pages discuss: 5120 / 14336 / 34816 for the
Quark dense linear in P1's maintainer question, and K-up 192 -> 512, V-up
512 -> 256 over 16 heads for the MLA absorbed projections in P3):

* activations ~ N(0, 1), optionally with 1% of the K channels (rounded,
  at least 1) scaled x20 as outliers;
* weights ~ N(0, 0.02); bias ~ N(0, 0.1);
* edge structure: per 1x32 block, exact-zero blocks (half of them holding
  -0.0), blocks whose amax is raised to a power of two, tie blocks (amax
  2^j plus elements on the seven E2M1 rounding midpoints scaled by
  2^(j-2)), and blocks with tiny negatives that round to -0.
"""

from __future__ import annotations

import numpy as np
import torch

ROLE_A, ROLE_W, ROLE_BIAS, ROLE_OUTLIER, ROLE_EDGE = 0, 1, 2, 3, 4

# Rounding midpoints of the E2M1 magnitudes (0, .5, 1, 1.5, 2, 3, 4, 6) and
# the magnitudes themselves: inputs that land exactly on them after the
# power-of-two block scaling exercise the tie rule.
_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
_ON_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def rng(seed: int, role: int, *dims: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(role), *[int(d) for d in dims]])


def to_bf16_bits(a) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16) via torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_to_torch_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bit patterns -> a CPU torch.bfloat16 tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def activations(M: int, K: int, seed: int, *, tag=(), outliers: bool = False,
                edge: bool = False) -> np.ndarray:
    """Activation matrix [M, K] as bf16 bits.  ``tag`` extends the rng key."""
    a = rng(seed, ROLE_A, M, K, *tag).standard_normal((M, K), dtype=np.float32)
    if outliers:
        n_out = max(1, int(round(0.01 * K)))
        ch = rng(seed, ROLE_OUTLIER, M, K, *tag).choice(K, size=n_out, replace=False)
        a[:, ch] *= np.float32(20.0)
    if edge:
        a = _edge_structure(a, rng(seed, ROLE_EDGE, M, K, *tag))
    return to_bf16_bits(a)


def weights(N: int, K: int, seed: int, *, tag=(), std: float = 0.02) -> np.ndarray:
    w = rng(seed, ROLE_W, N, K, *tag).standard_normal((N, K), dtype=np.float32)
    return to_bf16_bits(w * np.float32(std))


def bias(N: int, seed: int, *, tag=()) -> np.ndarray:
    b = rng(seed, ROLE_BIAS, N, *tag).standard_normal(N, dtype=np.float32)
    return to_bf16_bits(b * np.float32(0.1))


def _edge_structure(a: np.ndarray, r: np.random.Generator) -> np.ndarray:
    """Impose the edge-block categories on a [M, K] fp32 sample, per 1x32 block."""
    M, K = a.shape
    blk = a.reshape(M, K // 32, 32).copy()
    u = r.random((M, K // 32))
    for (m, c), cat in np.ndenumerate(u):
        v = blk[m, c]
        if cat < 1 / 8:                       # exact-zero block
            v[:] = 0.0
            if r.random() < 0.5:
                v[:] = -0.0
        elif cat < 2 / 8:                     # amax raised to a power of two
            i = int(np.argmax(np.abs(v)))
            p = np.float32(2.0) ** np.ceil(np.log2(np.abs(v[i])))
            v[i] = np.copysign(p, v[i])
        elif cat < 5 / 16:                    # tie block around amax = 2^j
            j = int(r.integers(-12, 13))
            unit = np.float32(2.0) ** (j - 2)
            vals = np.concatenate([_MIDPOINTS, _ON_GRID])
            pick = r.choice(vals, size=32)
            sign = np.where(r.random(32) < 0.5, -1.0, 1.0).astype(np.float32)
            v[:] = sign * pick * unit
            v[0] = np.float32(2.0) ** j * sign[0]
        elif cat < 6 / 16:                    # tiny negatives that round to -0
            amax = np.abs(v).max()
            idx = r.choice(32, size=4, replace=False)
            keep = int(np.argmax(np.abs(v)))
            idx = idx[idx != keep]
            v[idx] = -amax * np.float32(2.0) ** -7
    return blk.reshape(M, K)


def linear_problem(M: int, N: int, K: int, seed: int, *, outliers: bool = False,
                   with_bias: bool = False, edge: bool = False):
    """One W4A4 linear problem: dict with x [M,K], w [N,K], bias [N] or None."""
    return {
        "x": activations(M, K, seed, outliers=outliers, edge=edge),
        "w": weights(N, K, seed),
        "bias": bias(N, seed) if with_bias else None,
    }


def bmm_problem(B: int, M: int, N: int, K: int, seed: int):
    """One A16WFP4 BMM problem: x [B, M, K] bf16 bits, w [B, N, K] bf16 bits."""
    x = rng(seed, ROLE_A, B, M, N, K).standard_normal((B, M, K), dtype=np.float32)
    w = rng(seed, ROLE_W, B, N, K).standard_normal((B, N, K), dtype=np.float32)
    return {"x": to_bf16_bits(x), "w": to_bf16_bits(w * np.float32(0.02))}
