"""E4M3 codec (test oracle only).

DeepGEMM write-up, section 2.1: the FP8 format used for the forward pass has 4
exponent bits and 3 mantissa bits and tops out at 448.  Together with the
Triton-cutlass article's note that activations use E4M3, this fixes the OCP
"E4M3FN" layout: exponent bias 7, subnormals at exponent field 0, no infinity,
and S.1111.111 the only NaN.  Values are exact multiples of 2**-9; the largest
is 0x7E = 1.75 * 2**8 = 448.

``encode_e4m3`` rounds to nearest with ties to the even code and saturates at
+-448 (the format has no infinity; section 2.1's "overflow becomes infinity"
cannot happen in this layout, so an out-of-range magnitude is clamped - the
reading recorded for this step).  The sign of the input is kept, so -0.0 and
negative values that round to zero give 0x80.
"""

from __future__ import annotations

import numpy as np

from .minifloat import E4M3FN

#: all 254 finite codes (0x7F and 0xFF are NaN)
FINITE_E4M3_CODES = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def decode_e4m3(codes) -> np.ndarray:
    """uint8 codes -> exact fp64 values (NaN for 0x7F/0xFF)."""
    return E4M3FN.decode(np.asarray(codes, dtype=np.int64))


def encode_e4m3(t) -> np.ndarray:
    """fp32 values -> uint8 codes: round half to even, saturate to +-448."""
    t = np.asarray(t)
    if t.dtype != np.float32:
        raise TypeError("encode_e4m3 takes the fp32 quotient x / s")
    return E4M3FN.encode(t.astype(np.float64), overflow="saturate").astype(np.uint8)
