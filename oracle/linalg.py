"""W4A4 MXFP4 GEMM and A16WFP4 batched GEMM in fp64 (CPU oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

W4A4 GEMM.  P1 §Accuracy Tests states the property the method reaches: the
block-scaled FP4 GEMM gives the same output as a separately dequantised FP4
reference.  P2 §2 (apply_weights and the registered GEMM op) fixes the
operation: quantise activations per 1x32, multiply by the preshuffled [N, K]
weight as an NT product with output shape (M, N), then add the bias.  So the
oracle is that plain definition:
    y[m, n] = sum_k dq(A)[m, k] * dq(W)[n, k] + bias[n]
in fp64 (numpy matmul), then one round-to-nearest-even cast to bf16.  The
bias is added before the single cast (reading: a GEMM with an optional bias
rounds once; the pages add it after a bf16 GEMM, which rounds twice).

A16WFP4 BMM.  P3 §Motivation and §Modifications keep the absorbed MLA K/V
projection weights in packed MXFP4 and run the batched products on bf16
activations; the V-up result is written batch-major.  The oracle is
    O[b, m, n] = sum_k X[b, m, k] * dq(W)[b, n, k]
in fp64, X taken exactly from its bf16 bits, then one bf16 cast.  The
weight's 1x32 blocks run along the contraction axis K (reading: the pages do
not state the block axis; this matches the W4A4 weights).

Tolerance term.  ``abs_sum`` returns sum_k |a_k * b_k| per output element:
the GPU result before the bf16 cast must be within 2^-18 of that (plus
|bias|) of the fp64 value.

Pins (tests/test_oracle_linalg.py): exact ``fractions.Fraction`` brute force
on tiny shapes; the blockwise closed form sum over blocks of
2^(sa+sb-254) * (integer multiple of 1/4); a single block worked by hand;
the cross-path identity (an exactly MXFP4-representable X through the BMM
equals its quantised form through the GEMM); invariance under appended zero
blocks with 0x7F scales.
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, f64_to_bf16
from .quant import dequant, quant_1x32


def gemm_a4w4_from_quant(qa, sa, qw, sw, bias_bf16=None):
    """fp64 GEMM from quantised operands.

    qa [M, K/2], sa [M, K/32], qw [N, K/2], sw [N, K/32] (row-major scales),
    bias_bf16 None or uint16 [N].  Returns (y fp64 [M, N], abs_sum fp64 [M, N]).
    """
    a = dequant(qa, sa)
    w = dequant(qw, sw)
    y = a @ w.T
    s = np.abs(a) @ np.abs(w).T
    if bias_bf16 is not None:
        y = y + bf16_to_f64(bias_bf16)[None, :]
    return y, s


def gemm_a4w4(x_bf16, w_bf16, bias_bf16=None):
    """Whole W4A4 linear from bf16 inputs: quantise both, then the fp64 GEMM.

    x_bf16 uint16 [M, K], w_bf16 uint16 [N, K].  Returns (y fp64, abs_sum).
    """
    qa, sa = quant_1x32(x_bf16)
    qw, sw = quant_1x32(w_bf16)
    return gemm_a4w4_from_quant(qa, sa, qw, sw, bias_bf16)


def bmm_a16wfp4(x_bf16, qw, sw):
    """fp64 A16WFP4 BMM: x uint16 [B, M, K], qw [B, N, K/2], sw [B, N, K/32].

    Returns (O fp64 [B, M, N], abs_sum fp64 [B, M, N]).
    """
    x = bf16_to_f64(x_bf16)
    w = dequant(qw, sw)
    wt = np.swapaxes(w, 1, 2)
    return x @ wt, np.abs(x) @ np.abs(wt)


def to_bf16(y):
    """The single round-to-nearest-even cast of an fp64 result to bf16 bits."""
    return f64_to_bf16(y)
