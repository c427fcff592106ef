"""fp64 CPU oracle for softmax attention, forward and backward (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path must not.
"""
from .oracle import attn_bwd, attn_fwd, build, default_threads, run_workload  # noqa: F401
