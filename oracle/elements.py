"""The other MX element types: FP8 (E4M3, E5M2) and FP6 (E2M3, E3M2)
(oracle; test infrastructure only).

Source: "MXFP4", AI Wiki, §Place in the MX family: the MX v1.0 formats all use
32-element blocks and an E8M0 scale; MXFP8 has FP8 E5M2 or E4M3 elements and
MXFP6 FP6 E3M2 or E2M3 elements.  §Conversion rules: X is the largest power
of two not above the block's max |V_i| divided by the largest power of two the
element type can represent, each V_i / X is rounded to nearest-even and
clamped to the element's largest normal.

The pages name the element types only; their bit-level definitions are read
as OCP MX v1.0's (which the page cites): EkMm has k exponent bits with bias
2^(k-1) - 1, m mantissa bits and subnormals at exponent field 0;
  * E4M3: no infinities, S.1111.111 is NaN, largest normal S.1111.110 = 448;
  * E5M2: exponent field 11111 is Inf (mantissa 0) or NaN, largest normal 57344;
  * E2M3, E3M2 (FP6): every code is finite; largest normals 7.5 and 28.
(E2M1, FP4, keeps its own module: ``oracle.formats``.)

Storage (a reading; the hardware operand layout is checked against it on the
GPU): FP8 codes are one byte per element; FP6 codes are packed little-endian,
element i of a row at bits 6i .. 6i+5 of the row's bit string, so a 32-element
block fills 24 bytes.
"""

import numpy as np

from .formats import BLOCK

# name: (exponent bits, mantissa bits, largest finite magnitude code)
ELEMS = {
    "e4m3": (4, 3, 0x7E),
    "e5m2": (5, 2, 0x7B),
    "e2m3": (2, 3, 0x1F),
    "e3m2": (3, 2, 0x1F),
}


def elem_bits(elem):
    e, m, _ = ELEMS[elem]
    return 1 + e + m


def decode(codes, elem):
    """Decode integer codes (sign at bit e+m) to float64 with the usual
    floating-point rule: normal (1 + f/2^m) 2^(E - bias), subnormal E == 0:
    (f/2^m) 2^(1 - bias); E4M3's S.1111.111 is NaN; E5M2's top exponent is
    +-Inf (f == 0) or NaN."""
    e, m, _ = ELEMS[elem]
    bias = (1 << (e - 1)) - 1
    c = np.asarray(codes).astype(np.int64)
    s = (c >> (e + m)) & 1
    E = (c >> m) & ((1 << e) - 1)
    f = c & ((1 << m) - 1)
    mag = np.where(E == 0, np.ldexp(f / 2.0**m, 1 - bias), np.ldexp(1.0 + f / 2.0**m, E - bias))
    if elem == "e4m3":
        mag = np.where((E == 15) & (f == 7), np.nan, mag)
    if elem == "e5m2":
        mag = np.where(E == 31, np.where(f == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


def grid(elem):
    """The finite non-negative magnitudes in code order 0 .. largest."""
    return decode(np.arange(ELEMS[elem][2] + 1), elem)


def max_normal(elem):
    return float(grid(elem)[-1])


def emax(elem):
    """Exponent of the largest power of two the element type represents."""
    return int(np.floor(np.log2(max_normal(elem))))


def round_elem(v, elem, rounding="rne", r=None):
    """Round float32 values v (already divided by the block scale) to codes:
    lo <= |v| < hi neighbouring grid points, f = (|v| - lo) / (hi - lo);
    RNE: up iff f > 1/2 or (f == 1/2 and lo's code is odd); SR: up iff
    r < f 2^16; |v| at or above the largest normal saturates to it; the sign
    bit is kept (also for zero)."""
    e, m, top = ELEMS[elem]
    g = grid(elem)
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    sign = np.signbit(v).astype(np.int64)
    i = np.clip(np.searchsorted(g, a, side="right") - 1, 0, top - 1)
    lo, hi = g[i], g[i + 1]
    f = (a - lo) / (hi - lo)
    if rounding == "rne":
        up = (f > 0.5) | ((f == 0.5) & (i % 2 == 1))
    elif rounding in ("sr", "sr8"):
        if r is None:
            raise ValueError("stochastic rounding needs random bits r")
        up = np.asarray(r, dtype=np.float64) < f * (65536.0 if rounding == "sr" else 256.0)
    else:
        raise ValueError(f"unknown rounding {rounding!r}")
    idx = np.where(a >= g[-1], top, i + up.astype(np.int64))
    return (sign << (e + m)) | idx


def pack(codes, elem):
    """[R, K] codes -> [R, K * bits / 8] bytes (FP8: one byte each; FP6:
    element i at bits 6i .. 6i+5 of the row, little-endian)."""
    c = np.asarray(codes).astype(np.uint64)
    R, K = c.shape
    if elem_bits(elem) == 8:
        return c.astype(np.uint8)
    if K % 4:
        raise ValueError("FP6 rows must hold a multiple of 4 elements")
    # 4 codes -> 24 bits -> 3 bytes
    q = c.reshape(R, K // 4, 4)
    word = q[..., 0] | (q[..., 1] << np.uint64(6)) | (q[..., 2] << np.uint64(12)) | (q[..., 3] << np.uint64(18))
    out = np.empty((R, K // 4, 3), dtype=np.uint8)
    for b in range(3):
        out[..., b] = ((word >> np.uint64(8 * b)) & np.uint64(0xFF)).astype(np.uint8)
    return out.reshape(R, K * 3 // 4)


def unpack(packed, elem, K):
    """Inverse of ``pack``: [R, K * bits / 8] bytes -> [R, K] codes."""
    p = np.asarray(packed, dtype=np.uint8)
    R = p.shape[0]
    if elem_bits(elem) == 8:
        return p[:, :K].astype(np.int64)
    t = p[:, :K * 3 // 4].reshape(R, K // 4, 3).astype(np.uint64)
    word = t[..., 0] | (t[..., 1] << np.uint64(8)) | (t[..., 2] << np.uint64(16))
    out = np.empty((R, K // 4, 4), dtype=np.int64)
    for j in range(4):
        out[..., j] = ((word >> np.uint64(6 * j)) & np.uint64(0x3F)).astype(np.int64)
    return out.reshape(R, K)


def row_bytes(K, elem):
    return K * elem_bits(elem) // 8


def block_bits(elem):
    """Bits of one MX block: 32 elements plus the 8-bit scale."""
    return BLOCK * elem_bits(elem) + 8
