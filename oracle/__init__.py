"""CPU oracle for the SAW-INT4 KV-cache path and its controls (numpy, float32 IEEE).

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the product path. It shares no code
with the HIP library and imports nothing from it.

Parity pins (what fixes each function other than itself) are listed in
tests/test_oracle_pins.py; every function here is pinned.
"""
from .sawint4 import (  # noqa: F401
    F16_MAX, ROT_K, ROT_KV, ROT_NONE, c_h, decode_vectors, dequant_gather,
    dequant_exact, encode_vectors, fwht_blocks, mse, pack_nibbles,
    paged_decode_attention, quantize,
    quantize_append, quantize_with_scale, rotate, token_scale, unpack_nibbles,
)
from .controls import (  # noqa: F401
    cache_append, decode8_vectors, encode8_vectors, int8_append, int8_gather,
    quantize8_with_scale, token_scale8,
)
