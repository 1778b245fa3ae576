"""CPU oracle for the scattered mixture-of-experts hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product library imports, calls or
links this package; only the tests, the smoke check and the CPU-baseline leg
of the benchmark do.  It shares no code with the HIP path.

Sources (cited by page title and section):
  [PP]   ScatterMoE project page (sourcepulse.org), "How It Works" and
         "Highlighted Details".
  [RV1], [RV2], [RV3]
         Review page "Scattered Mixture-of-Experts Implementation", the
         Summary section of the first, second and third review.
  [ABS]  Catalogue record "Scattered Mixture-of-Experts Implementation",
         abstract.
  [ART]  Article "This Machine Learning Research Presents ScatterMoE: An
         Implementation of Sparse Mixture-of-Experts (SMoE) on GPUs", body,
         paragraphs 1-5.

Every function is pinned by a CPU test against something other than itself
(a library routine, a brute-force dense evaluation, autograd, finite
differences, invariants or a hand-worked example); see tests/test_oracle_*.
"""
from .smoe import *  # noqa: F401,F403
