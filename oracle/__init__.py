"""fp64 CPU oracle of the MoE expert layer (test infrastructure only).

Only tests, the package smoke check and the benchmark's CPU-baseline leg use
this package. The GPU library never imports it and shares no code with it.
"""
from . import moe_oracle  # noqa: F401
