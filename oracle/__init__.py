"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .kvq_oracle import (  # noqa: F401
    D_HEAD, GROUP, QMAX, BITS, levels,
    hadamard_rotation, rotate_rows, quantize_rows, pack_codes, unpack_codes,
    dequantize, quantize_cache, decode_attention, tie_distance,
)
