"""Block-scaled MXFP4 GEMM reference (oracle; test infrastructure only).

Source: "MXFP4", AI Wiki, §Conversion rules (dot products): a block dot
product is X(A) X(B) sum_i P_i(A) P_i(B); a longer dot product is the sum of
block dot products; the result should be float32 and internal precision and
order are left to the implementation.  The reference is therefore the plain
definition, evaluated exactly enough to judge any float32 implementation:

    ref[m, n] = sum_k a[m, k] * b[n, k]        (float64, dequantized operands)
    S[m, n]   = sum_k |a[m, k] * b[n, k]|      (the error scale)

with a, b the exactly decoded MXFP4 values (every one is a dyadic rational
that float64 holds exactly).  A NaN scale makes every output that its block
contributes to NaN ("MXFP4", AI Wiki, §Format specification: NaN scale
poisons the block).  ``block_dot_exact`` evaluates one dot product in exact
rational arithmetic, for the brute-force pins.
"""

from fractions import Fraction

import numpy as np

from . import elements
from .formats import BLOCK, e2m1_decode, e8m0_decode
from .quantize import unpack_nibbles


def _decode_f64(codes, scales, block, rows=None, elem="e2m1"):
    """Dequantize (optionally only some rows) to float64, no RHT."""
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    if rows is not None:
        rows = np.asarray(rows)
        codes = codes[rows]
        srows = rows // BLOCK if block == "2d" else rows
        sc = e8m0_decode(scales[srows])
    else:
        sc = e8m0_decode(scales)
        if block == "2d":
            sc = np.repeat(sc, BLOCK, axis=0)
    if elem == "e2m1":
        vals = e2m1_decode(unpack_nibbles(codes))
    else:
        K = codes.shape[1] * 8 // elements.elem_bits(elem)
        vals = elements.decode(elements.unpack(codes, elem, K), elem)
    with np.errstate(invalid="ignore"):
        return vals * np.repeat(sc, BLOCK, axis=1)


def dequant_f64(codes, scales, elem="e2m1", block="1d"):
    """The operand's exact values as float64 [rows, K] (no transform)."""
    return _decode_f64(codes, scales, block, None, elem)


def gemm_ref(a_codes, a_scales, b_codes, b_scales, a_block="1d", b_block="1d",
             rows=None, cols=None, a_elem="e2m1", b_elem="e2m1"):
    """Reference C = A * B^T for K-major MX operands A [M, K], B [N, K]
    (element types a_elem, b_elem; MXFP4 by default).

    rows/cols optionally restrict the output to a sample (index arrays).
    Returns (ref, S) as float64 arrays [len(rows), len(cols)].  A NaN or
    infinite element, like a NaN scale, makes its outputs NaN.
    """
    a = _decode_f64(a_codes, a_scales, a_block, rows, a_elem)
    b = _decode_f64(b_codes, b_scales, b_block, cols, b_elem)
    a = np.where(np.isinf(a), np.nan, a)
    b = np.where(np.isinf(b), np.nan, b)
    nan_a = np.isnan(a).any(axis=1)
    nan_b = np.isnan(b).any(axis=1)
    a0 = np.where(np.isnan(a), 0.0, a)
    b0 = np.where(np.isnan(b), 0.0, b)
    ref = a0 @ b0.T
    bound = np.abs(a0) @ np.abs(b0).T
    ref[nan_a, :] = np.nan
    ref[:, nan_b] = np.nan
    return ref, bound


def grouped_gemm_ref(a_codes, a_scales, offsets, b_codes, b_scales,
                     a_block="1d", b_block="2d", rows=None, cols=None, a_elem="e2m1", b_elem="e2m1"):
    """Reference for the MoE grouped GEMM: rows [off[e], off[e+1]) of A and of
    the output belong to expert e and use B[e] ([E, N, K/2] codes, per-expert
    scales).  rows (sorted or not) / cols restrict the output to a sample."""
    offsets = np.asarray(offsets, dtype=np.int64)
    M = int(offsets[-1])
    rows = np.arange(M) if rows is None else np.asarray(rows)
    N = np.asarray(b_codes).shape[1]
    cols = np.arange(N) if cols is None else np.asarray(cols)
    ref = np.empty((len(rows), len(cols)))
    bound = np.empty_like(ref)
    expert = np.searchsorted(offsets, rows, side="right") - 1
    for e in np.unique(expert):
        sel = np.nonzero(expert == e)[0]
        r, s = gemm_ref(a_codes, a_scales, b_codes[e], b_scales[e], a_block, b_block,
                        rows=rows[sel], cols=cols, a_elem=a_elem, b_elem=b_elem)
        ref[sel] = r
        bound[sel] = s
    return ref, bound


def block_dot_exact(a_codes, a_scale, b_codes, b_scale):
    """One block dot product X(A) X(B) sum_i P_i(A) P_i(B) in exact rationals.

    a_codes, b_codes: sequences of 4-bit codes of equal length (a multiple of
    32 is not required); a_scale, b_scale: E8M0 bytes (not 0xFF).
    """
    pa = [Fraction(float(v)) for v in e2m1_decode(np.asarray(a_codes))]
    pb = [Fraction(float(v)) for v in e2m1_decode(np.asarray(b_codes))]
    xa = Fraction(2) ** (int(a_scale) - 127)
    xb = Fraction(2) ** (int(b_scale) - 127)
    return xa * xb * sum(p * q for p, q in zip(pa, pb))
