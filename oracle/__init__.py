"""fp64 CPU oracle for attention: softmax forward, backward, ordered skipping, alpha-entmax (test
infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path must not.
"""
from .oracle import (attn_bwd, attn_fwd, attn_fwd_osk, build, default_threads, entmax_fwd,  # noqa: F401
                     run_workload)
