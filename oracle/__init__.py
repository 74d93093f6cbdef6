"""CPU oracle for the ReSpinQuant online path. TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the CPU-baseline leg of the
benchmark may import this package. The library's own code never does, and
this package imports nothing from the library: the two share no code. Their
only common source is ``synth`` (seeded random draws).

Sources are five AI-written summaries of the paper "ReSpinQuant: Efficient
Layer-Wise LLM Quantization via Subspace Residual Rotation Approximation"
(arXiv 2604.11080) on gist.science, in Chinese (zh), Italian (it), Dutch (nl),
Spanish (es) and French (fr). Citations name the page by its language and
the section of its technical summary, e.g. "zh §2.2".

What is computed (float64 unless the step fixes another precision):

offline (``prep``)
  Sylvester Walsh-Hadamard, Cayley transform, rotations R = H C(eps A),
  basis mismatch T = R_out^T R_in, SVD of dT = T - I, top-r basis U_r,
  Q_r = U_r^T T U_r, M = Q_r - I_r, per-output-channel weight quantisation.
online (``online``)
  projection p = h U_r, subspace transform c = p M, reprojection and
  residual h' = h + c U_r^T (rounded to the residual's storage type),
  RMSNorm, per-token symmetric quantisation, packing, integer GEMM,
  dequantisation, and the composition over one decoder layer's linears.

Every function is pinned by the CPU tests (``tests/test_oracle_*.py``)
against closed forms, invariants, special cases, brute force and the counts
the pages print. No function is left "parity unpinned".
"""
from . import numerics, packing, prep, online  # noqa: F401
