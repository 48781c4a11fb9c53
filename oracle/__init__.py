"""fp64 CPU oracle for the fused low-rank layer hot path.

TEST INFRASTRUCTURE: only the tests, the package entry point's smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path never does.
"""
from . import fsvd_oracle, loops  # noqa: F401
