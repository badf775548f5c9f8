"""MXFP4 element and scale formats (oracle; test infrastructure only).

Source: "MXFP4", AI Wiki, §Format specification — the parameter table
(E2M1: 1 sign, 2 exponent, 1 mantissa bit, bias 1, subnormals, no Inf/NaN;
E8M0: unsigned 8-bit biased exponent, bias 127, exponents -127..127, one NaN
code 0b11111111, no zero, no infinity; k = 32; 136 bits per block).

The E2M1 decode here is derived from the bit fields with the usual
floating-point decoding rule (normal: 2^(E-bias) * (1 + M/2); subnormal
E == 0: 2^(1-bias) * (M/2)).  The page's eight-row value table is *not* typed
in here: it is the pin that the test suite checks this derivation against.
"""

import numpy as np

BLOCK = 32                 # k, elements per MX block
E2M1_BIAS = 1
E8M0_BIAS = 127
E8M0_NAN = 0xFF


def e2m1_decode(codes):
    """Decode 4-bit E2M1 codes (ints 0..15, bit 3 = sign) to float64 values."""
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    normal = np.ldexp(1.0 + m / 2.0, (e - E2M1_BIAS).astype(np.int64))
    subnormal = np.ldexp(m / 2.0, 1 - E2M1_BIAS)
    mag = np.where(e == 0, subnormal, normal)
    return np.where(s == 1, -mag, mag)


# The eight non-negative magnitudes in code order 0..7, derived from the
# decoding rule above (pinned against the page's table in the tests).
E2M1_GRID = e2m1_decode(np.arange(8))


def e8m0_decode(codes):
    """Decode E8M0 scale bytes to float64: 2^(c - 127); code 0xFF is NaN."""
    c = np.asarray(codes).astype(np.int64)
    val = np.ldexp(1.0, np.where(c == E8M0_NAN, 0, c - E8M0_BIAS))
    return np.where(c == E8M0_NAN, np.nan, val)


def bf16_bits_to_f32(bits):
    """Widen bfloat16 bit patterns (uint16) to float32, exactly."""
    b = np.asarray(bits).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)
