"""Float64 CPU oracle for the POET-X layer -- test infrastructure only.

Only the tests, the smoke check and the bench's CPU-baseline leg use it; the
HIP library never calls it and shares no code with it.
"""
from .poetx_oracle import *  # noqa: F401,F403
