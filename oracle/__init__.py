"""fp64 CPU oracle for the MoDA forward and the depth-stream packer.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use it to check and to time against; the product path never
imports it.
"""
from .oracle import (  # noqa: F401
    moda_fwd,
    moda_fwd_rows,
    moda_bwd,
    moda_bwd_sampled,
    kv_project,
    pack_depth,
    append_depth_slot,
    default_threads,
)
