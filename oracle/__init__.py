"""CPU oracle for Gated DeltaNet chunked prefill -- TEST INFRASTRUCTURE ONLY.

Imported only by tests, the smoke check and the benchmark's CPU-baseline leg.
The GPU library shares no code with this package and never imports it.
"""
from .oracle import ref_fwd, ref_bwd, rel_l2, to_f64, default_threads  # noqa: F401
from .l2norm import L2_EPS, l2norm, l2norm_bwd, ref_bwd_l2, ref_fwd_l2  # noqa: F401
