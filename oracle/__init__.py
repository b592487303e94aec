"""fp64 CPU oracle for the GALE 1-bit routed-expert matmul.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark, never by the GPU library or its Python binding.
"""
from .gale_oracle import *  # noqa: F401,F403
from .gale_oracle import (  # noqa: F401
    hadamard, rotate, unpack_signs, decode_int4, outlier_triplets, dequantize, gemv,
    silu, ffn, route, moe, group_by_expert, packed_bytes, bits_per_weight,
    bits_per_weight_closed_form, rel_l2, popcount,
)
