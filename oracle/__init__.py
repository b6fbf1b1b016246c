"""CPU oracle of the MoE expert operation and of the step-time model.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the GPU library
(``expert_ffn_amd``) and never imports it.

* ``moe_oracle.c`` / ``ffn.py``: grouping, union count, requested bytes and the
  expert FFN, in double (Lan, arXiv:2610.34440, Section 1).
* ``reuse.py``: union X(n), reuse rho(n) and their window estimators on traces
  (Section 1 "Routing, union and reuse"; Appendix D.2 estimator).
* ``step_exact.py``: the step-time model, speedup condition, staircase, step
  points and reuse thresholds in exact rational arithmetic (Sections 3.1-3.4,
  Appendix B).
* ``fits.py``: the fits on chosen ids (Eq. (4), Eq. (E.1)), the bandwidth error
  and the Table 2 bounds (Sections 2, 3.5, 4; Appendix C).
* ``router.py``: the router ahead of the expert operation (Section 1): top-m
  logits, ties to the lower id, softmax over the selected.
"""
from .ffn import (  # noqa: F401
    build, route_group, union_count, union_count_batch, bytes_requested, expert_apply,
    moe_ffn_f64, moe_ffn, OR_OK, OR_E_INVAL, OR_E_DTYPE, OR_E_IDS,
)
