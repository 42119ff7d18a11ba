"""CPU fp64 oracle for absorbed MLA decode over a paged latent KV cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
CPU-baseline leg of the benchmark may import this package; the product path
(the HIP library and its Python binding) never does, and the two share no
code.  See ``oracle/mla_oracle.c`` for the definition it implements and the
passages of the pages it follows.
"""
from .oracle import (  # noqa: F401
    BF16,
    E4M3FN,
    F64,
    build,
    decode,
    e4m3fn_to_float64,
    bf16_bits_to_float64,
)
