"""MXFP4 quantizer and dequantizer (oracle; test infrastructure only).

Sources:
  * "MXFP4", AI Wiki, §Conversion rules: the reference scale is the largest
    power of two not above the block's max |V_i|, divided by 4 (the largest
    power of two in E2M1); elements V_i/X are quantized to FP4 with
    round-to-nearest-ties-to-even and clamped (saturated) to +-6.
  * "MXFP4", AI Wiki, §Clipping in the reference algorithm: the shared
    exponent is floor(log2(amax)) - 2, the scaled block max lies in [4, 8), and
    values that scale into (6, 8) clip to 6 (worked example: amax 7.5 -> X = 1,
    stored as 6).
  * "MXFP4", AI Wiki, §Format specification: E8M0 scale (bias 127, range
    -127..127, NaN code 0xFF poisons the whole block), 32-element blocks.
  * "MXFP4", AI Wiki, §Use in models / gpt-oss: two FP4 values per byte,
    block scales stored apart, blocks along the last dimension.
  * "Training an MoE LLM in MXFP4", summary: hybrid 1D/2D block quantization,
    randomized Hadamard transform, stochastic rounding.
  * Two other scale rules, both named on the MXFP4 page:
    - "round_up" (§Clipping in the reference algorithm, the rule credited to
      NVIDIA's NVFP4 pretraining report): the decode scale amax/6 rounded up to
      a power of two, so that no element saturates.
    - "prescale_3_4" (§Training with MXFP4, the table's Tseng, Yu, Park
      row): the inputs are multiplied by 3/4 before quantizing so that nothing
      clips.  Read as: the
      reference rule's scale of the block as given, and every element times
      3/4 (one float32 multiply) before the division by it.

Steps per block, in the order they are taken (float32 where stated):
  1. x = float32(source) (bf16 widens exactly).
  2. optional RHT along the blocking axis (see ``oracle.rht``).
  3. amax = max |y_i| over the block (1D: 32 elements along K; 2D: the 32x32
     tile).  A block holding any NaN or +-Inf gets scale 0xFF and all codes 0.
  4. E = floor(log2 amax) taken exactly from the float32 exponent (subnormals
     included); e = clamp(E - 2, -127, 127); amax == 0 gives e = -127.
     round_up: e = the smallest integer with amax <= 6 * 2^e, clamped the
     same way.  Scale byte = e + 127.
  5. prescale_3_4 only: y_i = float32(0.75 * y_i).
     v_i = float32(y_i * 2^-e): one float32 multiply (exact unless the result
     is a float32 subnormal, which is rounded to nearest even and never flushed).
  6. Round |v_i| onto the grid {0, .5, 1, 1.5, 2, 3, 4, 6}: |v| >= 6 saturates
     to 6; otherwise lo <= |v| < hi are the neighbouring grid points and
     f = (|v| - lo)/(hi - lo) (exact).  RNE: up iff f > 1/2, or f == 1/2 and
     lo's code is odd (ties go to the even mantissa bit).  SR: up iff
     r < f * 2^16 for the element's 16 random bits r (``oracle.philox``);
     "sr8": up iff r < f * 2^8 for its 8 random bits (bias at most 2^-8 of
     the step: P(up) = ceil(256 f) / 256).
  7. code = sign(v) << 3 | magnitude index; the sign of a zero is kept.
  8. two codes per byte, element 2j in the low nibble of byte j.

Readings of points the pages leave open: "flush values below the smallest
subnormal to zero" is taken as what RNE on the full grid already does
(|v| <= 0.25 -> 0); the sign of zero is kept; amax == 0 uses the lowest scale;
NaN/Inf blocks use the NaN scale; SR saturates deterministically above 6.
"""

import numpy as np

from . import elements
from .formats import BLOCK, E2M1_GRID, E8M0_BIAS, E8M0_NAN, e2m1_decode, e8m0_decode
from .philox import sr_bits8, sr_bits16
from .rht import rht_forward_f32, rht_inverse_f32


def shared_exponent(amax, emax=2):
    """e = clamp(floor(log2 amax) - emax, -127, 127) for float32 amax >= 0
    (finite); amax == 0 maps to -127.  emax is the exponent of the largest
    power of two of the element type (2 for E2M1).  floor(log2) comes from
    frexp, which is exact for normal and subnormal float32 inputs."""
    a = np.asarray(amax, dtype=np.float32)
    _, ex = np.frexp(a)                      # a = m * 2^ex, m in [0.5, 1)
    e = (ex.astype(np.int64) - 1) - emax
    e = np.clip(e, -127, 127)
    return np.where(a == 0, -127, e)


def round_up_exponent(amax, top=6.0, emax=2):
    """The smallest integer e with amax <= top * 2^e (top: the element type's
    largest normal, 6 for E2M1), clamped to [-127, 127], for finite float32
    amax >= 0 (amax == 0 maps to -127).  The candidate floor(log2 amax) - emax
    from frexp is tried first and raised by one when top * 2^e still falls
    short; both sides are exact in float64."""
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    _, ex = np.frexp(a)
    e = ex.astype(np.int64) - 1 - emax
    e = np.where(a > np.ldexp(top, e.astype(np.int32)), e + 1, e)
    e = np.clip(e, -127, 127)
    return np.where(a == 0, -127, e)


SCALE_MODES = ("floor", "round_up", "prescale_3_4")


def round_e2m1(v, rounding="rne", r=None):
    """Round float32 values v (already divided by the block scale) to E2M1 codes."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    sign = np.signbit(v).astype(np.int64)
    grid = E2M1_GRID                                   # [0, .5, 1, 1.5, 2, 3, 4, 6]
    i = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, 6)
    lo = grid[i]
    hi = grid[np.minimum(i + 1, 7)]
    f = (a - lo) / (hi - lo)
    if rounding == "rne":
        up = (f > 0.5) | ((f == 0.5) & (i % 2 == 1))
    elif rounding in ("sr", "sr8"):
        if r is None:
            raise ValueError("stochastic rounding needs random bits r")
        up = np.asarray(r, dtype=np.float64) < f * (65536.0 if rounding == "sr" else 256.0)
    else:
        raise ValueError(f"unknown rounding {rounding!r}")
    idx = np.where(a >= 6.0, 7, i + up.astype(np.int64))
    return (sign << 3) | idx


def pack_nibbles(codes):
    """[R, K] codes 0..15 -> [R, K/2] uint8, element 2j in the low nibble."""
    c = np.asarray(codes).astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """[R, K/2] uint8 -> [R, K] codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0x0F
    out[:, 1::2] = p >> 4
    return out


def quantize(x, axis="last", block="1d", rounding="rne", rht_mask=None,
             seed=0, offset=0, row_index=None, K_total=None, scale_mode="floor", elem="e2m1",
             stats=None):
    """Quantize a 2-D float array to MXFP4.

    axis="last": blocks along the last dim, output [R, C] with K = C.
    axis="dim0": blocks along dim 0, output is the quantized transpose [C, R]
                 (K = R), still with blocks along its last dim.
    block="1d": one scale per 32 elements along K, scales [rows_out, K/32].
    block="2d": one scale per 32x32 tile, scales [rows_out/32, K/32].
    Returns (codes uint8 [rows_out, K/2], scales uint8).

    row_index / K_total let a caller quantize a sample of output rows (or of
    source columns, for axis="dim0") of a larger tensor: they give the global
    output-row numbers and the global K used in the stochastic-rounding element
    index p = row * K + k.  They change nothing else.
    scale_mode: "floor" (the reference rule), "round_up" or "prescale_3_4".
    elem: "e2m1" (MXFP4, two codes per byte) or another MX element type of
    ``oracle.elements`` ("e4m3", "e5m2": one byte per element; "e2m3",
    "e3m2": 6-bit codes packed little-endian); the scale takes that type's
    largest power of two and the elements its grid (§Conversion rules).
    stats: a dict that, when given, receives stats["clipped"], the number of
    elements of finite blocks whose scaled value (step 5) lies above the
    element type's largest normal, i.e. that saturate in step 6 (§Clipping in
    the reference algorithm: with the reference rule, values scaling into
    (6, 8) clip to 6).
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("quantize expects a 2-D array")
    if axis == "dim0":
        x = x.T
    elif axis != "last":
        raise ValueError(f"unknown axis {axis!r}")
    rows, K = x.shape
    if elem != "e2m1" and elem not in elements.ELEMS:
        raise ValueError(f"unknown element type {elem!r}")
    if scale_mode not in SCALE_MODES:
        raise ValueError(f"unknown scale_mode {scale_mode!r}")
    if K % BLOCK:
        raise ValueError("the blocking dimension must be a multiple of 32")
    if block == "2d" and rows % BLOCK:
        raise ValueError("2-D blocks need rows_out to be a multiple of 32")
    nkb = K // BLOCK

    y = x.reshape(rows, nkb, BLOCK)
    if rht_mask is not None:
        y = rht_forward_f32(y, rht_mask)

    with np.errstate(invalid="ignore", over="ignore"):
        finite = np.isfinite(y)
        absy = np.where(finite, np.abs(y), np.float32(0))
        if block == "1d":
            amax = absy.max(axis=-1)                                  # [rows, nkb]
            bad = ~finite.all(axis=-1)
        elif block == "2d":
            amax = absy.reshape(rows // BLOCK, BLOCK, nkb, BLOCK).max(axis=(1, 3))
            bad = ~finite.reshape(rows // BLOCK, BLOCK, nkb, BLOCK).all(axis=(1, 3))
        else:
            raise ValueError(f"unknown block {block!r}")

        if elem == "e2m1":
            e = round_up_exponent(amax) if scale_mode == "round_up" else shared_exponent(amax)
        else:
            em = elements.emax(elem)
            e = (round_up_exponent(amax, elements.max_normal(elem), em) if scale_mode == "round_up"
                 else shared_exponent(amax, em))
        scales = np.where(bad, E8M0_NAN, e + E8M0_BIAS).astype(np.uint8)

        if block == "2d":                       # per-element view of the tile scale
            e_el = np.repeat(e, BLOCK, axis=0)
            bad_el = np.repeat(bad, BLOCK, axis=0)
        else:
            e_el, bad_el = e, bad
        if scale_mode == "prescale_3_4":
            y = (np.float32(0.75) * y).astype(np.float32)
        factor = np.ldexp(np.float32(1.0), (-e_el).astype(np.int32)).astype(np.float32)
        v = (y * factor[..., None]).astype(np.float32)

        r = None
        if rounding in ("sr", "sr8"):
            ridx = np.arange(rows) if row_index is None else np.asarray(row_index)
            kt = K if K_total is None else int(K_total)
            p = (ridx.astype(np.uint64)[:, None] * np.uint64(kt)
                 + np.arange(K, dtype=np.uint64)[None, :])
            bits = sr_bits16 if rounding == "sr" else sr_bits8
            r = bits(p, seed, offset).reshape(rows, nkb, BLOCK)
        codes = round_e2m1(v, rounding, r) if elem == "e2m1" else elements.round_elem(v, elem, rounding, r)
        codes = np.where(bad_el[..., None], 0, codes)
        if stats is not None:
            top = np.float32(6.0) if elem == "e2m1" else np.float32(elements.max_normal(elem))
            stats["clipped"] = int(np.count_nonzero((np.abs(v) > top) & ~bad_el[..., None]))
    if elem != "e2m1":
        return elements.pack(codes.reshape(rows, K), elem), scales
    return pack_nibbles(codes.reshape(rows, K)), scales


def clip_count(x, axis="last", block="1d", rht_mask=None, scale_mode="floor", elem="e2m1"):
    """Clipping statistic of one quantization (§Clipping in the reference
    algorithm): how many elements of x saturate at the element type's largest
    normal when x is quantized with these settings (the rounding mode does
    not matter: every mode saturates the same values).  Blocks holding NaN or
    Inf count nothing (their codes are all zero).  With the round-up rule or
    the 3/4 prescale the count is 0 by construction."""
    st = {}
    quantize(x, axis=axis, block=block, rht_mask=rht_mask, scale_mode=scale_mode, elem=elem, stats=st)
    return st["clipped"]


def quantize_gather(x, rows, rounding="rne", rht_mask=None, seed=0, offset=0,
                    scale_mode="floor"):
    """Quantize the gathered rows x[rows[i]] (1-D blocks along the last dim):
    the MoE front end of "Training an MoE LLM in MXFP4" (summary), where each
    token's activations are quantized once per expert it is routed to, with
    the output row number i in the stochastic-rounding element index.  An index
    outside [0, R) stands for no source row: its output row holds NaN blocks
    (scale 0xFF, codes 0), the format's only way to mark invalid data
    ("MXFP4", AI Wiki, §Format specification: the NaN scale poisons the block).
    """
    x = np.asarray(x, dtype=np.float32)
    rows = np.asarray(rows, dtype=np.int64)
    R, C = x.shape
    valid = (rows >= 0) & (rows < R)
    g = np.zeros((rows.shape[0], C), dtype=np.float32)
    g[valid] = x[rows[valid]]
    codes, scales = quantize(g, rounding=rounding, rht_mask=rht_mask, seed=seed, offset=offset,
                             scale_mode=scale_mode)
    codes[~valid] = 0
    scales[~valid] = E8M0_NAN
    return codes, scales


def quantize_scatter(x, dest, k, rows_out, out_codes=None, out_scales=None, rht_mask=None,
                     scale_mode="floor"):
    """The MoE front end from the token side: row t of x is quantized once
    (1-D blocks along the last dim, RNE) and written to output rows
    dest[t*k + j], j < k; destinations outside [0, rows_out) are skipped and
    rows no destination names keep out_codes / out_scales (zeros if not
    given).  RNE codes depend only on the row's values, so this is the
    quantization of the routed rows ("Training an MoE LLM in MXFP4", summary)
    computed once per token."""
    x = np.asarray(x, dtype=np.float32)
    dest = np.asarray(dest, dtype=np.int64).reshape(x.shape[0], k)
    codes, scales = quantize(x, rounding="rne", rht_mask=rht_mask, scale_mode=scale_mode)
    oc = np.zeros((rows_out, codes.shape[1]), np.uint8) if out_codes is None else np.array(out_codes, np.uint8)
    os_ = np.zeros((rows_out, scales.shape[1]), np.uint8) if out_scales is None else np.array(out_scales, np.uint8)
    for t in range(x.shape[0]):
        for j in range(k):
            d = dest[t, j]
            if 0 <= d < rows_out:
                oc[d] = codes[t]
                os_[d] = scales[t]
    return oc, os_


def transpose_2d(codes, scales, elem="e2m1"):
    """Transpose of an operand quantized with 2-D (32x32) blocks: [R, C] ->
    [C, R].  A 32x32 tile shares one scale whichever way it is read, so element
    (c, r) of the result carries the code of element (r, c) and tile (j, i)
    the scale byte of tile (i, j); nothing is re-rounded.  This is the reading
    behind the 2-D weight blocks of the hybrid 1D/2D recipe ("Training an MoE
    LLM in MXFP4", summary): one quantization of W serves X W and, transposed,
    dY W^T.  Other element types (elem) transpose their codes the same way."""
    if elem == "e2m1":
        c = unpack_nibbles(codes)
    else:
        cd = np.asarray(codes)
        c = elements.unpack(cd, elem, cd.shape[1] * 8 // elements.elem_bits(elem))
    s = np.asarray(scales, dtype=np.uint8)
    if c.shape[0] % BLOCK or c.shape[1] % BLOCK:
        raise ValueError("2-D blocks need both dimensions to be multiples of 32")
    if s.shape != (c.shape[0] // BLOCK, c.shape[1] // BLOCK):
        raise ValueError("expected one scale per 32x32 tile")
    ct = np.ascontiguousarray(c.T)
    packed = pack_nibbles(ct) if elem == "e2m1" else elements.pack(ct, elem)
    return packed, np.ascontiguousarray(s.T)


def dequantize(codes, scales, block="1d", inverse_rht_mask=None, dtype=np.float32, elem="e2m1"):
    """Decode MXFP4: value = E2M1(code) * 2^(scale - 127); scale 0xFF makes the
    whole block NaN.  Optional inverse RHT (float32, canonical order).  Other
    element types (elem) decode their codes with ``oracle.elements``."""
    if elem == "e2m1":
        vals = e2m1_decode(unpack_nibbles(codes))                   # float64 [R, K]
    else:
        K = np.asarray(codes).shape[1] * 8 // elements.elem_bits(elem)
        vals = elements.decode(elements.unpack(codes, elem, K), elem)
    rows, K = vals.shape
    sc = e8m0_decode(scales)
    if block == "2d":
        sc = np.repeat(sc, BLOCK, axis=0)
    sc = np.repeat(sc, BLOCK, axis=1)
    with np.errstate(invalid="ignore", over="ignore"):
        x = vals * sc
        if inverse_rht_mask is not None:
            x32 = x.astype(np.float32).reshape(rows, K // BLOCK, BLOCK)
            return rht_inverse_f32(x32, inverse_rht_mask).reshape(rows, K)
        return x.astype(dtype)
