"""CPU oracle for the MoE layout / dispatch / combine path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package; the HIP library shares no code with it.
"""
from . import moe_oracle  # noqa: F401
from .moe_oracle import *  # noqa: F401,F403
