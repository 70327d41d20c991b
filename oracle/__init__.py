"""CPU oracle (test infrastructure only; never imported by the library).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
"""
from .aqlm_oracle import (  # noqa: F401
    bits_per_weight, check_format, decode, decode_rows, forward, forward_rows,
    packed_bits_per_weight, product, unpack_codes, within_tolerance,
)
from . import encoder_oracle  # noqa: F401
