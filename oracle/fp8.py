"""fp8 (OCP e4m3) decoding for the fp8 prefill (oracle; test infrastructure
only).

e4m3 byte: sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent 0
encodes subnormals m/8 * 2^-6; 0x7F and 0xFF are NaN; there is no infinity,
so the largest finite value is 0x7E = 1.75 * 2^8 = 448.  The fp8 inputs of
the attention are these exact values times a per-tensor descale factor; the
oracle attention then runs in fp64 on them (the fp8 path asked about in
[flashinfer#724], closing questions).
"""

import numpy as np


def e4m3_decode(codes):
    """float64 values of e4m3 bytes (any shape)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)
