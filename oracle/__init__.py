"""Float64 CPU oracle for the paged KV-cache hot path (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
this package; the library and its binding never import it.
"""
from .pagedattn import *  # noqa: F401,F403
