"""fp64 CPU oracle for the CODA GEMM-epilogue path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use it.
"""
from . import coda_oracle  # noqa: F401
