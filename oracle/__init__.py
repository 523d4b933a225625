"""CPU oracle for the NVFP4 block-scaled grouped GEMM (test infrastructure only:
imported by the tests, the smoke check and the benchmark's CPU-baseline leg)."""
from .nvfp4_oracle import *  # noqa: F401,F403
from . import nvfp4_oracle  # noqa: F401
