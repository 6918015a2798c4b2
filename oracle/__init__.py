"""CPU oracle for one GPU's share of a sparse MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP library (no kernels, headers,
helpers, tables or constants); both sides read their inputs from the seeded
generator in ``workload``.
"""
from .moe_oracle import *  # noqa: F401,F403
