"""CPU oracle for Gated DeltaNet chunked prefill -- TEST INFRASTRUCTURE ONLY.

Imported only by tests, the smoke check and the benchmark's CPU-baseline leg.
The GPU library shares no code with this package and never imports it.
"""
from .oracle import ref_fwd, ref_bwd, rel_l2, to_f64, default_threads  # noqa: F401
