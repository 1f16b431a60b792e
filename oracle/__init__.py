"""CPU oracle for the raw-token hashed n-gram embedding.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this package.  It shares no
code with the HIP path.
"""
from .engram_oracle import (Oracle, build, build_all, default_oracle,  # noqa: F401
                            openmp_oracle)
