"""fp64 CPU oracle for Tensor Product Attention.  Test infrastructure only:
imported by the tests, the smoke check and the benchmark's CPU baseline, never
by the product path."""
from .tpa_oracle import (  # noqa: F401
    Dims, project, rope, rope_angles, positions, rotate_factors, cache_new, cache_append,
    reconstruct, queries, attend_head, prefill, decode, layer_forward,
)
