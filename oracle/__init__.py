"""CPU oracle for InfLLM v2 block-sparse attention.

TEST INFRASTRUCTURE ONLY: only the tests, the package smoke check and the benchmark's
CPU-baseline leg may import this package.  The HIP library never uses it.
"""
from . import infllm2_oracle, brute  # noqa: F401
