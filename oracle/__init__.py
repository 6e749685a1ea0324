"""CPU float64 oracle for the sparse-MoE FFN forward.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.
"""
from .moe_oracle import *  # noqa: F401,F403
from .philox import gumbel_noise, gumbel_uniform, gumbel_words, philox4x32_10  # noqa: F401
