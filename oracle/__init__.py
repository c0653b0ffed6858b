"""CPU oracle for the NVFP4 paged KV cache — test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the library never does.
"""
from .nvfp4_oracle import *  # noqa: F401,F403
