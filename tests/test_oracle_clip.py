"""Pins for the oracle's clipping statistic (``oracle.clip_count``).

"MXFP4", AI Wiki, §Clipping in the reference algorithm: under the reference
scale rule the shared exponent is floor(log2 amax) - 2, the scaled block
maximum can reach just below 8, and values scaling into (6, 8) clip to 6 (a
block maximum of 7.5 gets scale 1 and is stored as 6); about 3 % of entries
clip on typical matrices; rounding the scale up to the next power of two
leaves nothing saturated, and so does the 3/4 prescale (§Training with
MXFP4, Tseng, Yu, Park).  The brute force below counts in exact float64
arithmetic against the threshold top * 2^e, a formulation independent of the
oracle's scaled float32 values.
"""
import math
import zlib

import numpy as np
import pytest

import oracle
from golden_io import params
from oracle import elements

ELEMS = ["e2m1", "e4m3", "e5m2", "e2m3", "e3m2"]
TOP = {"e2m1": 6.0, "e4m3": 448.0, "e5m2": 57344.0, "e2m3": 7.5, "e3m2": 28.0}
EMAX = {"e2m1": 2, "e4m3": 8, "e5m2": 15, "e2m3": 2, "e3m2": 4}


def _bruteforce(x, axis, block, elem):
    """Clipped elements under the reference rule, block by block in Python
    floats: e = clamp(floor(log2 amax) - emax, -127, 127) from frexp, clipped
    iff |y| > top * 2^e (all exact in float64)."""
    y = np.asarray(x, dtype=np.float32)
    if axis == "dim0":
        y = y.T
    rows, K = y.shape
    n = 0
    rstep = 32 if block == "2d" else 1
    for r0 in range(0, rows, rstep):
        for k0 in range(0, K, 32):
            blk = [float(v) for v in y[r0:r0 + rstep, k0:k0 + 32].ravel()]
            if any(not math.isfinite(v) for v in blk):
                continue
            amax = max(abs(v) for v in blk)
            if amax == 0.0:
                continue
            _, ex = math.frexp(amax)
            e = min(max(ex - 1 - EMAX[elem], -127), 127)
            lim = TOP[elem] * 2.0 ** e
            n += sum(1 for v in blk if abs(v) > lim)
    return n


def _data(rng, rows, cols):
    """Log-uniform magnitudes over many binades with random signs, so block
    maxima fall all over their binade; a few exact powers of two and zeros."""
    mag = np.exp2(rng.uniform(-20, 20, (rows, cols)))
    x = (mag * rng.choice([-1.0, 1.0], (rows, cols))).astype(np.float32)
    x[rng.random((rows, cols)) < 0.02] = 0.0
    x[0, :32] = np.float32(4.0)
    return x


def test_worked_example_7_5_clips():
    """A block whose largest magnitude is 7.5 gets scale 1 and 7.5 saturates
    (§Clipping in the reference algorithm); a maximum of exactly 6 or 4 does
    not clip."""
    p = params("clipping_example.txt")
    amax = float(p["amax"])
    x = np.full((1, 32), 1.0, dtype=np.float32)
    x[0, 5] = amax
    assert oracle.clip_count(x) == 1
    codes, scales = oracle.quantize(x)
    assert int(scales[0, 0]) == 127
    assert (int(oracle.unpack_nibbles(codes)[0, 5]) & 7) == 7      # stored as 6
    for m in (6.0, 4.0):
        x[0, 5] = m
        assert oracle.clip_count(x) == 0


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("axis,block", [("last", "1d"), ("last", "2d"), ("dim0", "1d"), ("dim0", "2d")])
def test_clip_count_bruteforce(elem, axis, block):
    rng = np.random.default_rng(zlib.crc32(f"{elem}{axis}{block}".encode()))
    x = _data(rng, 64, 96)
    n = oracle.clip_count(x, axis=axis, block=block, elem=elem)
    assert n == _bruteforce(x, axis, block, elem)
    assert n > 0


def test_nan_and_inf_blocks_count_nothing():
    x = np.full((2, 64), 7.5, dtype=np.float32)
    x[:, 0] = 1.0
    x[0, 3] = np.nan
    x[1, 40] = np.inf
    # row 0: block 0 holds NaN (nothing), block 1 is all 7.5 (scale 1: 32 clip)
    # row 1: block 0 clips 31 (the 1.0 does not), block 1 holds Inf (nothing)
    assert oracle.clip_count(x) == 32 + 31


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("rht", [None, 0x5A5AC3C3])
def test_round_up_and_prescale_never_clip(elem, rht):
    """Round-up scales and the 3/4 prescale leave nothing saturated (the
    page's stated purpose of both), on data whose block maxima sit just below
    the top of their binade, where the reference rule clips most."""
    rng = np.random.default_rng(7)
    x = _data(rng, 64, 128)
    x[:, ::32] = np.float32(1.99) * np.exp2(rng.integers(-10, 10, (64, 4))).astype(np.float32)
    assert oracle.clip_count(x, rht_mask=rht, elem=elem) > 0
    for mode in ("round_up", "prescale_3_4"):
        for axis in ("last", "dim0"):
            for block in ("1d", "2d"):
                assert oracle.clip_count(x, axis=axis, block=block, rht_mask=rht, scale_mode=mode, elem=elem) == 0


def test_clipped_fraction_near_three_percent():
    """About 3 % of entries clip on typical matrices (§Clipping in the
    reference algorithm): 1-5 % on Gaussian and Student-t data, with and
    without the transform."""
    rng = np.random.default_rng(11)
    for x in (rng.standard_normal((256, 1024)), rng.standard_t(3, (256, 1024))):
        x = x.astype(np.float32)
        for rht in (None, 0x1234ABCD):
            frac = oracle.clip_count(x, rht_mask=rht) / x.size
            assert 0.01 < frac < 0.05, frac


def test_clipped_elements_store_the_largest_code():
    """Every clipped element is stored as the largest magnitude (the clip is
    a saturation): with the transform, count <= the number of largest codes."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((128, 256)).astype(np.float32)
    n = oracle.clip_count(x, rht_mask=0xF0F0F0F0)
    codes, _ = oracle.quantize(x, rht_mask=0xF0F0F0F0)
    top = int(np.count_nonzero((oracle.unpack_nibbles(codes) & 7) == 7))
    assert 0 < n <= top
