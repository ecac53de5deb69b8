"""Plain CPU reference for the ternary rotated-basis linear y = W(Rx).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this package.  The HIP library never
calls it, and it shares no code, table or helper with the HIP sources.

Everything is computed in float64 with numpy, written to be read against the
pages rather than to be fast.  See ``oracle.ternary`` for the functions and the
passages each one follows.
"""
from .ternary import (  # noqa: F401
    GROUP, BLOCK, B3_BYTES_PER_GROUP,
    pack_2bit, unpack_2bit, pack_base3, unpack_base3, packed_row_bytes, bits_per_weight,
    hadamard, sign_vector, rotate, dequantize, gemv, gemm, rel_err, normwise_err,
    TERNARY_CANDIDATES, rotate_weights, f64_to_f16_bits, ternarize, quantize_weights,
)
