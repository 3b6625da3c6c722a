"""fp64 CPU reference for the attention forward and backward passes.

TEST INFRASTRUCTURE ONLY: the checker the GPU kernels are compared against.
Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it.  It shares no code with the GPU library.
"""
from .oracle import (OracleLib, attention_bwd, attention_fwd, build_oracle, dropout_multiplier,  # noqa: F401
                     oracle_threads, philox4x32_10)
