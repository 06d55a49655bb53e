"""fp64 CPU oracle of the hybrid K4V4/FP16 decode-attention path.

Test infrastructure only: imported by the test suite, the package smoke check
and the benchmark's CPU-baseline leg, never by the GPU library.
"""
from . import hq_oracle  # noqa: F401
