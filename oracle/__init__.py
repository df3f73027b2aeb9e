"""CPU oracle (float64 numpy) for the NVFP4 routed-expert MoE projection.

Test infrastructure only: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.
"""
from .nvfp4_oracle import *  # noqa: F401,F403
