"""Pins for the oracle quantizer.

Each pin comes from the pages or from mathematics independent of the oracle's
own formulation:
  * the reference scale rule and its clipping ("MXFP4", AI Wiki, §Conversion
    rules; §Clipping in the reference algorithm, including the 7.5 -> 6 example
    and the ~3 % clipped estimate);
  * RNE / saturation by brute force: nearest of the page's eight E2M1 values,
    ties to the code with mantissa bit 0 (the page's bit table);
  * stochastic rounding is unbiased with the binomial variance (closed form);
  * dim-0 blocking equals last-dim blocking of the transpose; 2-D tiles take
    their scale from the tile maximum.
"""
import math

import numpy as np
import pytest

import oracle
from golden_io import e2m1_table, params
from oracle.formats import BLOCK


def _nearest_code_bruteforce(a):
    """|v| -> magnitude code by exhaustive distance over the page's table;
    ties go to the code whose mantissa bit (bit 0) is 0; saturate above 6."""
    table = e2m1_table()
    best = None
    for code, val, _ in table:
        d = abs(a - val)
        key = (d, code & 1)
        if best is None or key < best[0]:
            best = (key, code)
    return best[1]


def _scale_of_block(codes, scales, col):
    return float(oracle.e8m0_decode(scales[0, col // 32]))


# ---------------------------------------------------------------- scale rule
def test_worked_clipping_example():
    p = params("clipping_example.txt")
    amax = float(p["amax"])
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = amax
    x[0, 1] = 1.0
    codes, scales = oracle.quantize(x)
    assert float(oracle.e8m0_decode(scales[0, 0])) == float(p["scale"])
    deq = oracle.dequantize(codes, scales)
    assert deq[0, 0] == float(p["stored"])
    assert deq[0, 1] == 1.0


def test_shared_exponent_closed_form_and_block_max_band():
    rng = np.random.default_rng(1)
    mags = np.exp(rng.uniform(-80, 80, size=20000)).astype(np.float32)
    mags = mags[(mags > 0) & np.isfinite(mags)]
    e = oracle.shared_exponent(mags)
    expect = np.array([math.floor(math.log2(float(m))) - 2 for m in mags])
    assert np.array_equal(e, np.clip(expect, -127, 127))
    ratio = mags.astype(np.float64) / np.ldexp(1.0, e)
    inrange = (e > -127)
    assert np.all((ratio[inrange] >= 4.0) & (ratio[inrange] < 8.0))


def test_shared_exponent_exact_powers_and_subnormals():
    for k in range(-149, 128):
        a = np.float32(2.0 ** k)
        assert oracle.shared_exponent(a) == max(k - 2, -127)
        below = np.nextafter(a, np.float32(0))
        if below > 0:
            assert oracle.shared_exponent(below) == max(k - 3, -127)
    assert oracle.shared_exponent(np.float32(0)) == -127


def test_scale_rule_on_random_blocks_matches_definition():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((40, 32 * 6)) * np.exp(rng.uniform(-20, 20, (40, 1)))).astype(np.float32)
    codes, scales = oracle.quantize(x)
    for r in range(x.shape[0]):
        for b in range(6):
            amax = np.abs(x[r, b * 32:(b + 1) * 32]).max()
            # largest power of two not above amax, divided by 4
            p2 = 2.0 ** math.floor(math.log2(float(amax)))
            assert float(oracle.e8m0_decode(scales[r, b])) == p2 / 4


def test_clipped_fraction_soft_statistic():
    """About 3 % of entries land in the clip band (6, 8) ("MXFP4", AI Wiki,
    §Clipping); accept 1-5 % on Gaussian and Student-t data."""
    p = params("clipping_example.txt")
    lo, hi = float(p["clip_band_low"]), float(p["clip_band_high"])
    rng = np.random.default_rng(3)
    for x in (rng.standard_normal((512, 1024)), rng.standard_t(3, (512, 1024))):
        x = x.astype(np.float32)
        codes, scales = oracle.quantize(x)
        sc = np.repeat(oracle.e8m0_decode(scales), 32, axis=1)
        v = np.abs(x) / sc
        frac = np.mean((v > lo) & (v < hi))
        assert 0.01 < frac < 0.05


# ---------------------------------------------------------------- rounding
def _grid_probe_values():
    """Every grid point, every midpoint, +-1..3 float32 ulps around each, the
    clip band, and the subnormal region."""
    grid = [v for _, v, _ in e2m1_table()]
    pts = set(grid)
    for a, b in zip(grid[:-1], grid[1:]):
        pts.add((a + b) / 2)
    pts.update([6.5, 7.0, 7.5, 7.99, 0.1, 0.25, 0.2, 0.3, 0.74, 0.76, 1e-30, 1e-40])
    out = set()
    for p in pts:
        f = np.float32(p)
        out.add(float(f))
        up, dn = f, f
        for _ in range(3):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(0))
            out.add(float(up))
            out.add(float(dn))
    return sorted(v for v in out if v < 8.0)


def test_rne_bruteforce_over_grid_midpoints_and_clip_band():
    vals = np.array(_grid_probe_values(), dtype=np.float32)
    got = oracle.round_e2m1(vals, "rne")
    for v, c in zip(vals, got):
        assert c == _nearest_code_bruteforce(float(v)), float(v)
    got_neg = oracle.round_e2m1(-vals, "rne")
    assert np.array_equal(got_neg, got | 8)


def test_rne_specific_ties():
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for v, expect in ties.items():
        c = oracle.round_e2m1(np.float32(v), "rne")
        assert oracle.e2m1_decode(c) == expect, v


def test_signed_zero_and_saturation():
    c = oracle.round_e2m1(np.array([-0.0, 0.0, -0.1, 1e9, -1e9], dtype=np.float32), "rne")
    assert list(c) == [8, 0, 8, 7, 15]


def test_nonfinite_and_zero_blocks():
    x = np.zeros((3, 64), dtype=np.float32)
    x[1, 3] = np.nan
    x[2, 40] = np.inf
    x[2, 0] = 1.0
    x[1, 33] = -2.0
    codes, scales = oracle.quantize(x)
    assert scales[0, 0] == 0 and scales[0, 1] == 0        # amax 0 -> lowest scale
    assert scales[1, 0] == 0xFF and scales[2, 1] == 0xFF
    assert scales[1, 1] == 126                            # amax 2 -> e = -1
    assert np.all(oracle.unpack_nibbles(codes)[1, :32] == 0)
    assert np.all(oracle.unpack_nibbles(codes)[2, 32:] == 0)
    deq = oracle.dequantize(codes, scales)
    assert np.isnan(deq[1, :32]).all() and np.isnan(deq[2, 32:]).all()
    assert deq[1, 33] == -2.0 and deq[2, 0] == 1.0


def test_dequantize_error_bound_unclipped():
    """|x - deq(q(x))| <= half a grid step at that magnitude times the scale,
    except in the clip band where it is |x| - 6X."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((128, 256)).astype(np.float32)
    codes, scales = oracle.quantize(x)
    deq = oracle.dequantize(codes, scales).astype(np.float64)
    sc = np.repeat(oracle.e8m0_decode(scales), 32, axis=1)
    v = np.abs(x) / sc
    step = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    err = np.abs(x - deq) / sc
    clip = v > 6
    assert np.all(err[~clip] <= step[~clip] / 2)
    assert np.allclose(err[clip], v[clip] - 6.0)


def test_subnormal_scaled_value_not_flushed():
    """A float32 product landing in the subnormal range is rounded, not flushed:
    its sign survives (-0 code) and in SR it can still round up with r = 0."""
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = np.float32(2.0 ** 120)
    x[0, 1] = -np.float32(2.0 ** -10)          # v = -2^-128, a float32 subnormal
    codes, scales = oracle.quantize(x)
    c = oracle.unpack_nibbles(codes)[0]
    assert c[1] == 8
    r = np.zeros(32, dtype=np.uint32)
    v = np.zeros(32, dtype=np.float32)
    v[1] = np.float32(-(2.0 ** -128))
    assert oracle.round_e2m1(v, "sr", r)[1] == 9      # r = 0 < f * 2^16 > 0


# ---------------------------------------------------------------- layouts
def test_nibble_order_low_first():
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 4.0      # scale 1 -> code 6
    x[0, 1] = 1.0      # code 2
    codes, scales = oracle.quantize(x)
    assert codes[0, 0] == 0x26


def test_dim0_equals_transpose_last_rne_and_sr():
    rng = np.random.default_rng(5)
    x = rng.standard_t(3, (96, 64)).astype(np.float32)
    for kw in ({}, {"rounding": "sr", "seed": 123456789, "offset": 7},
               {"rht_mask": 0xA5A5F00F}, {"block": "2d"}):
        a = oracle.quantize(x, axis="dim0", **kw)
        b = oracle.quantize(np.ascontiguousarray(x.T), axis="last", **kw)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_2d_scale_is_tile_max():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 96)).astype(np.float32)
    x[5, 70] = 300.0
    codes, scales = oracle.quantize(x, block="2d")
    assert scales.shape == (2, 3)
    for tr in range(2):
        for tc in range(3):
            amax = np.abs(x[tr * 32:(tr + 1) * 32, tc * 32:(tc + 1) * 32]).max()
            assert float(oracle.e8m0_decode(scales[tr, tc])) == 2.0 ** math.floor(math.log2(amax)) / 4
    # every element decodes against its tile's scale
    deq = oracle.dequantize(codes, scales, block="2d")
    assert abs(deq[5, 70] - 256.0) < 1e-9       # 300 / 64 = 4.69 -> 4 -> 256


def test_2d_transpose_consistency_rne():
    rng = np.random.default_rng(8)
    w = rng.standard_normal((64, 96)).astype(np.float32)
    c1, s1 = oracle.quantize(w, axis="dim0", block="2d")        # quantized W^T
    c2, s2 = oracle.quantize(w, axis="last", block="2d")        # quantized W
    d1 = oracle.dequantize(c1, s1, block="2d")
    d2 = oracle.dequantize(c2, s2, block="2d")
    assert np.array_equal(s1, s2.T)
    assert np.array_equal(d1, d2.T)


# ---------------------------------------------------------------- stochastic rounding
@pytest.mark.parametrize("v", [0.1, 0.3, 0.6, 1.2, 1.7, 2.25, 3.9, 4.5, 5.99])
def test_sr_unbiased_with_binomial_variance(v):
    n = 200_000
    rng = np.random.default_rng(int(v * 1000))
    r = rng.integers(0, 65536, size=n).astype(np.uint32)
    vals = np.full(n, v, dtype=np.float32)
    got = oracle.e2m1_decode(oracle.round_e2m1(vals, "sr", r))
    grid = [g for _, g, _ in e2m1_table()]
    lo = max(g for g in grid if g <= v)
    hi = min(g for g in grid if g > v)
    assert set(np.unique(got)) <= {lo, hi}
    sigma = math.sqrt((float(np.float32(v)) - lo) * (hi - float(np.float32(v))))
    tol = 5 * sigma / math.sqrt(n) + (hi - lo) * 2.0 ** -16
    assert abs(got.mean() - float(np.float32(v))) <= tol
    assert abs(got.var() - sigma ** 2) <= 0.05 * sigma ** 2 + 1e-6


def test_sr_quantize_unbiased_end_to_end():
    """Mean over many Philox offsets of the SR-dequantized tensor -> x."""
    rng = np.random.default_rng(9)
    x = (rng.uniform(-5.9, 5.9, (4, 32))).astype(np.float32)
    x[:, 0] = 5.95                          # pin the scale to 1 in every block
    acc = np.zeros_like(x, dtype=np.float64)
    n = 3000
    for off in range(n):
        c, s = oracle.quantize(x, rounding="sr", seed=42, offset=off)
        acc += oracle.dequantize(c, s).astype(np.float64)
    mean = acc / n
    # each element's sd <= max step / 2 = 1; 5-sigma bound
    assert np.max(np.abs(mean - x)) <= 5 * 1.0 / math.sqrt(n) + 2 * 2.0 ** -16


# ---------------------------------------------------------------- 8-bit draws
def _exact_fraction(v):
    """(lower grid index, exact fraction f) of a positive float32 v below 6,
    from the page's table."""
    from fractions import Fraction
    grid = [g for _, g, _ in e2m1_table()]
    i = max(k for k, g in enumerate(grid) if g <= v)
    return i, (Fraction(float(v)) - Fraction(grid[i])) / (Fraction(grid[i + 1]) - Fraction(grid[i]))


def test_sr8_threshold_bruteforce():
    """8-bit stochastic rounding: up iff r < f * 2^8, checked at the draws
    T - 1, T, T + 1 around T = floor(256 f) for fractions with and without an
    exact 8-bit representation, both signs."""
    rng = np.random.default_rng(51)
    vals = [np.float32(v) for v in rng.uniform(0.01, 5.99, 300)]
    vals += [np.float32(v) for v in (0.125, 0.25 + 0.5 / 256, 1.5 + 0.5 * 3 / 8, 3.5, 5.0 + 2.0 * 7 / 256)]
    for v in vals:
        i, f = _exact_fraction(v)
        if f == 0:
            continue
        t = int(f * 256)
        for r in (t - 1, t, t + 1):
            if not 0 <= r < 256:
                continue
            up = r < f * 256
            code = int(oracle.round_e2m1(np.float32([v]), "sr8", np.uint32([r]))[0])
            assert code == i + int(up), (float(v), r)
            assert int(oracle.round_e2m1(np.float32([-v]), "sr8", np.uint32([r]))[0]) == code | 8


def test_sr8_is_sr16_at_scaled_draws():
    """Rounding with an 8-bit draw r equals 16-bit stochastic rounding with the
    draw 256 r (256 r < f 2^16 exactly when r < f 2^8): the identity that lets
    a 16-bit implementation serve both."""
    rng = np.random.default_rng(52)
    v = rng.uniform(-6.5, 6.5, 200_000).astype(np.float32)
    r = rng.integers(0, 256, v.shape).astype(np.uint32)
    assert np.array_equal(oracle.round_e2m1(v, "sr8", r), oracle.round_e2m1(v, "sr", r * 256))


@pytest.mark.parametrize("v", [0.1, 0.3, 1.2, 1.7, 2.25, 3.9, 5.99])
def test_sr8_bias_at_most_a_256th_of_the_step(v):
    """P(up) = ceil(256 f) / 256 in closed form, so the mean is off v by less
    than 2^-8 of the step (above it), and the variance is binomial; checked over
    n Philox draws through the quantizer's own bit mapping."""
    import math
    x = np.float32(v)
    i, f = _exact_fraction(x)
    grid = [g for _, g, _ in e2m1_table()]
    lo, hi = grid[i], grid[i + 1]
    n = 1 << 18
    r = oracle.sr_bits8(np.arange(n, dtype=np.uint64), 1234, 0)
    got = oracle.e2m1_decode(oracle.round_e2m1(np.full(n, x), "sr8", r))
    pu = math.ceil(float(f) * 256) / 256
    mean_exact = lo + pu * (hi - lo)
    assert 0 <= mean_exact - float(x) < (hi - lo) / 256
    sigma = (hi - lo) * math.sqrt(pu * (1 - pu))
    assert abs(got.mean() - mean_exact) <= 5 * sigma / math.sqrt(n) + 1e-12
    assert abs(got.var() - sigma ** 2) <= 0.05 * sigma ** 2 + 1e-9


def test_sr8_dim0_equals_transpose_last():
    rng = np.random.default_rng(53)
    x = rng.standard_normal((64, 96)).astype(np.float32)
    kw = dict(rounding="sr8", seed=9, offset=2, rht_mask=0x13572468)
    c0, s0 = oracle.quantize(x, axis="dim0", **kw)
    c1, s1 = oracle.quantize(np.ascontiguousarray(x.T), **kw)
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)


def test_row_sampling_matches_full_tensor():
    """Quantizing a sample of rows with their global row numbers reproduces
    those rows of the full result (stochastic rounding included)."""
    rng = np.random.default_rng(10)
    x = rng.standard_normal((96, 64)).astype(np.float32)
    kw = dict(rounding="sr", seed=77, offset=3, rht_mask=0x0F0F00FF)
    full_c, full_s = oracle.quantize(x, **kw)
    rows = np.array([95, 0, 41])
    c, s = oracle.quantize(x[rows], row_index=rows, **kw)
    assert np.array_equal(c, full_c[rows]) and np.array_equal(s, full_s[rows])
    fc, fs = oracle.quantize(x, axis="dim0", **kw)
    cols = np.array([5, 63, 32])
    c, s = oracle.quantize(x[:, cols], axis="dim0", row_index=cols, **kw)
    assert np.array_equal(c, fc[cols]) and np.array_equal(s, fs[cols])


def test_gather_rows_are_quantized_under_their_output_row_number():
    """quantize_gather: output row i is source row rows[i] quantized with i as
    its row number in the stochastic-rounding index (checked row by row with
    the row-sampling form, itself pinned above); the identity gather equals the
    plain quantizer; out-of-range indices give NaN blocks that dequantize to
    NaN ("MXFP4", AI Wiki, §Format specification)."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((20, 96)).astype(np.float32)
    kw = dict(rounding="sr", seed=5, offset=9, rht_mask=0x00FF0F0F)
    ident = np.arange(20)
    gc, gs = oracle.quantize_gather(x, ident, **kw)
    fc, fs = oracle.quantize(x, **kw)
    assert np.array_equal(gc, fc) and np.array_equal(gs, fs)
    rows = np.array([3, 3, 19, -1, 0, 20, 7])
    gc, gs = oracle.quantize_gather(x, rows, **kw)
    for i, r in enumerate(rows):
        if 0 <= r < 20:
            c, s = oracle.quantize(x[r:r + 1], row_index=[i], K_total=96, **kw)
            assert np.array_equal(gc[i:i + 1], c) and np.array_equal(gs[i:i + 1], s)
        else:
            assert np.all(gc[i] == 0) and np.all(gs[i] == 0xFF)
            assert np.all(np.isnan(oracle.dequantize(gc[i:i + 1], gs[i:i + 1])))
    # the same source row under two output rows: equal scales, and equal codes
    # under RNE (SR draws differ with the output row number)
    rc, rs = oracle.quantize_gather(x, rows)
    assert np.array_equal(rc[0], rc[1]) and np.array_equal(rs[0], rs[1])


# ---------------------------------------------------------------- scale variants
def _round_up_exponent_bruteforce(amax):
    """Smallest integer e in [-127, 127] with amax <= 6 * 2^e, by search
    (exact rational arithmetic through Python floats: 6 * 2^e is exact)."""
    for e in range(-127, 128):
        if amax <= 6.0 * 2.0 ** e:
            return e
    return 127


def test_round_up_scale_is_smallest_power_of_two_without_saturation():
    """round_up: the decode scale amax/6 rounded up to a power of two ("MXFP4",
    AI Wiki, §Clipping in the reference algorithm), by brute force over all
    exponents, including the boundary amax = 1.5 * 2^k where amax/6 is itself
    a power of two, and the clamped ends."""
    p = params("scale_variants.txt")
    top = float(p["round_up_max_scaled"])
    rng = np.random.default_rng(21)
    mags = [float(np.float32(v)) for v in
            np.ldexp(rng.uniform(1.0, 2.0, 3000), rng.integers(-140, 128, 3000))]
    for k in range(-149, 128):
        b = np.float32(1.5 * 2.0 ** k) if k < 127 else np.float32(2.0 ** 127)
        if b == 0 or not np.isfinite(b):
            continue
        mags += [float(b), float(np.nextafter(b, np.float32(np.inf))),
                 float(np.nextafter(b, np.float32(0)))]
    mags += [float(np.finfo(np.float32).max), float(np.float32(2.0 ** -149))]
    for m in mags:
        x = np.zeros((1, 32), dtype=np.float32)
        x[0, 5] = -m
        codes, scales = oracle.quantize(x, scale_mode="round_up")
        e = _round_up_exponent_bruteforce(m)
        assert int(scales[0, 0]) == e + 127, m
        if e > -127:
            assert m / 2.0 ** e <= top and m / 2.0 ** e > top / 2
    # the boundary: scaled max exactly 6 stays at 6, one ulp above moves a binade
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 1.5
    c, s = oracle.quantize(x, scale_mode="round_up")
    assert oracle.e8m0_decode(s[0, 0]) == 0.25 and oracle.dequantize(c, s)[0, 0] == 1.5
    x[0, 0] = np.nextafter(np.float32(1.5), np.float32(2))
    c, s = oracle.quantize(x, scale_mode="round_up")
    assert oracle.e8m0_decode(s[0, 0]) == 0.5


def test_round_up_never_saturates_and_worst_case_binades():
    """With round_up no element scales above 6, so RNE codes are the nearest
    grid point by brute force with no clipping; the worst case (amax just
    above 6 * 2^k) leaves the 4 and 6 magnitudes unused, log2(3/0.5) of
    log2(6/0.5) binades ("MXFP4", AI Wiki, §Clipping in the reference
    algorithm: about 2.58 of 3.58)."""
    p = params("scale_variants.txt")
    rng = np.random.default_rng(22)
    x = (rng.standard_t(3, (24, 32 * 4)) * np.exp(rng.uniform(-6, 6, (24, 1)))).astype(np.float32)
    codes, scales = oracle.quantize(x, scale_mode="round_up")
    c = oracle.unpack_nibbles(codes)
    sc = np.repeat(oracle.e8m0_decode(scales), 32, axis=1)
    for r in range(x.shape[0]):
        for k in range(x.shape[1]):
            v = abs(float(x[r, k])) / float(sc[r, k])
            assert v <= 6.0
            assert c[r, k] & 7 == _nearest_code_bruteforce(v), (r, k, v)
            assert (c[r, k] >> 3) == int(np.signbit(x[r, k]))
    worst = np.zeros((1, 32), dtype=np.float32)
    worst[0, :] = np.linspace(-1, 1, 32, dtype=np.float32) * np.nextafter(np.float32(6 * 2.0 ** 3),
                                                                           np.float32(np.inf))
    wc, ws = oracle.quantize(worst, scale_mode="round_up")
    used = set(np.abs(oracle.dequantize(wc, ws)[0] / oracle.e8m0_decode(ws[0, 0])).tolist())
    unused = [float(t) for t in p["round_up_worst_unused_magnitudes"].split()]
    assert max(used) == 3.0 and not (set(unused) & used)
    assert abs(math.log2(6 / 0.5) - float(p["fp4_binades"])) < 0.01
    assert abs(math.log2(max(used) / 0.5) - float(p["round_up_worst_binades"])) < 0.01


def test_prescale_keeps_reference_scale_and_nothing_clips():
    """prescale_3_4: the scale is the reference rule's (largest power of two
    not above amax, over 4), the elements are 3/4 of the inputs, so the scaled
    maximum lies in [3, 6) and no element clips (the table row for Tseng, Yu,
    Park in "MXFP4", AI Wiki, §Training with MXFP4); codes are the
    brute-force nearest grid point of fl32(0.75 x) / X."""
    p = params("scale_variants.txt")
    f = np.float32(p["prescale_factor"])
    rng = np.random.default_rng(23)
    x = (rng.standard_t(3, (24, 32 * 4)) * np.exp(rng.uniform(-6, 6, (24, 1)))).astype(np.float32)
    codes, scales = oracle.quantize(x, scale_mode="prescale_3_4")
    c = oracle.unpack_nibbles(codes)
    for r in range(x.shape[0]):
        for b in range(4):
            blk = x[r, b * 32:(b + 1) * 32]
            X = 2.0 ** math.floor(math.log2(float(np.abs(blk).max()))) / 4
            assert float(oracle.e8m0_decode(scales[r, b])) == X
            v = np.abs((f * blk).astype(np.float32)).astype(np.float64) / X
            assert 3.0 <= v.max() < 6.0
            for k in range(32):
                assert c[r, b * 32 + k] & 7 == _nearest_code_bruteforce(v[k])


def test_clipped_fraction_is_zero_under_both_variants():
    """The reference rule clips a few percent of entries into the (6, 8) band
    ("MXFP4", AI Wiki, §Clipping); both variants exist to clip none."""
    p = params("clipping_example.txt")
    lo = float(p["clip_band_low"])
    f = float(params("scale_variants.txt")["prescale_factor"])
    rng = np.random.default_rng(24)
    x = rng.standard_t(3, (256, 1024)).astype(np.float32)
    for mode, mult in (("round_up", 1.0), ("prescale_3_4", f)):
        codes, scales = oracle.quantize(x, scale_mode=mode)
        sc = np.repeat(oracle.e8m0_decode(scales), 32, axis=1)
        assert np.mean(np.abs(x.astype(np.float64)) * mult / sc > lo) == 0.0


@pytest.mark.parametrize("mode,mult", [("round_up", 1.0), ("prescale_3_4", 0.75)])
def test_sr_unbiased_under_variants_where_floor_is_biased(mode, mult):
    """Nothing saturates under either variant, so stochastic rounding is
    unbiased for every element, the clipped maximum included: the mean over
    2048 seeds of the decoded block is mult * x within 5 standard errors
    (binomial variance <= step^2/4).  The reference rule loses the same
    property on the clipped element (7.5 -> always 6)."""
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :] = np.linspace(-7.5, 7.5, 32, dtype=np.float32)
    n = 2048
    acc = np.zeros(32)
    for seed in range(n):
        c, s = oracle.quantize(x, rounding="sr", seed=seed, offset=3, scale_mode=mode)
        acc += oracle.dequantize(c, s)[0]
    mean = acc / n
    target = (np.float32(mult) * x[0]).astype(np.float64)
    X = float(oracle.e8m0_decode(s[0, 0]))
    se = 2.0 * X / 2 / math.sqrt(n)
    assert np.all(np.abs(mean - target) <= 5 * se + 1e-12)
    cf, sf = oracle.quantize(x, rounding="sr", seed=0, offset=3)
    assert oracle.dequantize(cf, sf)[0, -1] == 6.0


def test_gather_passes_scale_mode():
    rng = np.random.default_rng(25)
    x = rng.standard_normal((10, 64)).astype(np.float32)
    rows = np.array([9, 2, 2, 0])
    for mode in ("round_up", "prescale_3_4"):
        gc, gs = oracle.quantize_gather(x, rows, scale_mode=mode)
        fc, fs = oracle.quantize(x[rows], scale_mode=mode)
        assert np.array_equal(gc, fc) and np.array_equal(gs, fs)
    with pytest.raises(ValueError):
        oracle.quantize(x, scale_mode="ceil")


# ---------------------------------------------------------------- 2-D transpose
def test_transpose_2d_is_quantizing_along_the_other_axis():
    """transpose_2d of W quantized along its last dim in 32x32 tiles equals W
    quantized along dim 0 in 32x32 tiles (RNE, no transform): a tile's scale is
    the same in both orientations and each element rounds alone.  Decoding
    commutes with it, twice is the identity, and 1-D layouts are refused."""
    rng = np.random.default_rng(41)
    for R, C in ((32, 32), (96, 160), (160, 64)):
        w = (rng.standard_t(3, (R, C)) * np.exp(rng.uniform(-4, 4, (R // 32, 1)).repeat(32, 0)))
        w = w.astype(np.float32)
        lc, ls = oracle.quantize(w, block="2d")
        dc, ds = oracle.quantize(w, axis="dim0", block="2d")
        tc, ts = oracle.transpose_2d(lc, ls)
        assert tc.shape == (C, R // 2) and ts.shape == (C // 32, R // 32)
        assert np.array_equal(tc, dc) and np.array_equal(ts, ds)
        assert np.array_equal(oracle.dequantize(tc, ts, "2d"), oracle.dequantize(lc, ls, "2d").T)
        bc, bs = oracle.transpose_2d(tc, ts)
        assert np.array_equal(bc, lc) and np.array_equal(bs, ls)
    c1, s1 = oracle.quantize(np.ones((32, 64), np.float32))
    with pytest.raises(ValueError):
        oracle.transpose_2d(c1, s1)


@pytest.mark.parametrize("elem", ["e4m3", "e5m2", "e2m3", "e3m2"])
def test_transpose_2d_other_element_types(elem):
    """The same pin for MXFP8 / MXFP6: transposing the last-dim 32x32-tile
    quantization gives the dim-0 one; twice is the identity."""
    rng = np.random.default_rng(43)
    w = (rng.standard_normal((96, 160)) * np.exp(rng.uniform(-3, 3, (3, 1)).repeat(32, 0))).astype(np.float32)
    lc, ls = oracle.quantize(w, block="2d", elem=elem)
    dc, ds = oracle.quantize(w, axis="dim0", block="2d", elem=elem)
    tc, ts = oracle.transpose_2d(lc, ls, elem)
    assert np.array_equal(tc, dc) and np.array_equal(ts, ds)
    bc, bs = oracle.transpose_2d(tc, ts, elem)
    assert np.array_equal(bc, lc) and np.array_equal(bs, ls)


def test_scatter_equals_gather_with_the_inverse_index():
    """Top-k routing: every output row is named by exactly one (token, slot)
    pair, so the scatter form (each token quantized once, stored k times)
    must give the gathered form's bytes with the inverse index, for RNE with
    and without the transform and in every scale mode; a destination outside
    the output is skipped and an unnamed row keeps its old bytes."""
    rng = np.random.default_rng(77)
    T, k, C = 12, 3, 96
    x = (rng.standard_normal((T, C)) * np.exp(rng.uniform(-3, 3, (T, 1)))).astype(np.float32)
    perm = rng.permutation(T * k)                 # output row of (token t, slot j) = perm[t*k + j]
    inv = np.empty(T * k, np.int64)
    inv[perm] = np.arange(T * k) // k             # token of each output row
    for mask, mode in [(None, "floor"), (0x5A5A1234, "round_up"), (None, "prescale_3_4")]:
        sc, ss = oracle.quantize_scatter(x, perm, k, T * k, rht_mask=mask, scale_mode=mode)
        gc, gs = oracle.quantize_gather(x, inv, rht_mask=mask, scale_mode=mode)
        np.testing.assert_array_equal(sc, gc)
        np.testing.assert_array_equal(ss, gs)
    dest = perm.copy()
    dest[4] = T * k + 7                          # outside: skipped
    old_c = np.full((T * k, C // 2), 0xA5, np.uint8)
    old_s = np.full((T * k, C // 32), 0x11, np.uint8)
    sc, ss = oracle.quantize_scatter(x, dest, k, T * k, old_c, old_s)
    assert np.all(sc[perm[4]] == 0xA5) and np.all(ss[perm[4]] == 0x11)
    qc, qs = oracle.quantize(x)
    np.testing.assert_array_equal(sc[perm[5]], qc[5 // k])
    np.testing.assert_array_equal(ss[perm[5]], qs[5 // k])
