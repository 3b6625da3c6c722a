"""fp64 CPU reference for the attention forward pass.

TEST INFRASTRUCTURE ONLY: the checker the GPU kernels are compared against.
Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it.  It shares no code with the GPU library.
"""
from .oracle import (OracleLib, attention_fwd, build_oracle, dropout_multiplier, oracle_threads,  # noqa: F401
                     philox4x32_10)
