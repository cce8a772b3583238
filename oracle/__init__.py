"""CPU oracle (test infrastructure only; never imported by the product path)."""

from .convrot_oracle import *  # noqa: F401,F403
from .convrot_oracle import (  # noqa: F401
    REGULAR, RANDOMIZED, QMAX, h4, regular_rotation, sylvester,
    randomized_block, rotate64, rotate, quantize_rows, code_values, pack,
    int_gemm, int_gemm_bruteforce, epilogue64, bf16_round, linear,
    linear_unquantized64, routes_to_fallback,
)
