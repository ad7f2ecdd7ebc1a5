"""fp64 CPU oracle for FusedKV reconstruction-layer attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.
"""
from .oracle import (attend, build, cache_capacity, cache_reads, num_threads,  # noqa: F401
                     row_index, VANILLA, LITE, FUSEDKV)
