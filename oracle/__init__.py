"""CPU oracle for the W4A4 MXFP4 linear and the A16WFP4 batched GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package.  The product path (the HIP library and its Python binding) never
touches it, and this package imports nothing from the product path.  The two
sides share no code; the only module both use is the seeded input generator,
which holds none of the method's arithmetic.

Sources the oracle follows (cited by tag in every docstring):

* P1 -- web page "[AMD] Add opt-in AITER ASM FP4 GEMM for Quark dense linear"
  (sgl-project/sglang pull request 39598).  Sections: Motivation,
  Modifications, Accuracy Tests.
* P2 -- web page "[sglang] SGLang, AMD GPU에서 Quark 모델의 FP4 GEMM 성능 최적화:
  AITER ASM 활용" (analysis of the same pull request, with its code diff).
  Sections: "코드 분석 / 2. AITER ASM FP4 GEMM 통합" (the scheme diff: scale
  swizzle, activation-scale padding, apply_weights) and
  "3. CPU Unit 테스트".
* P3 -- web page "[AMD] [GLM5] use tuned MXFP4 kernels for MLA absorbed BMM"
  (sgl-project/sglang pull request 34317).  Sections: Motivation,
  Modifications.
* OCP-MX -- the Open Compute Project "OCP Microscaling Formats (MX)
  Specification", version 1.0: the E2M1 element format, the E8M0 scale
  format, and the conversion of a vector of scalars into one MX block.  The
  pages name these formats but never define their arithmetic, so the public
  specification is the reading taken for it.

Modules:

* :mod:`oracle.formats` -- E2M1 / E8M0 / bf16 decoding and fp64 -> bf16
  round-to-nearest-even.
* :mod:`oracle.quant` -- per-1x32 MXFP4 quantisation and dequantisation.
* :mod:`oracle.layout` -- this library's own scale and weight layouts
  (index maps plus padding), and the pages' prior-art scale tile order.
* :mod:`oracle.linalg` -- the W4A4 GEMM and the A16WFP4 BMM in fp64, and the
  per-element tolerance term sum |a_i * b_i|.

Parity status per function is stated in each module header.  One quantity is
"parity unpinned": the internal precision of the hardware's scaled FP4 dot
product, which is not a function of this oracle and is only measured against
the tolerance.
"""

from . import formats, quant, layout, linalg  # noqa: F401
