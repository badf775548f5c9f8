"""Pins for the oracle's other MX element types (FP8 E4M3/E5M2, FP6 E2M3/E3M2).

  * the page's MX family table (element widths, block size, scale type);
  * FP8 decoding and round-to-nearest-even against torch's own float8_e4m3fn
    and float8_e5m2 types (a library implementation of the same OCP formats)
    over every code and over grid midpoints, ties and random values;
  * FP6 rounding by brute force over the decoded grid;
  * the page's scale rule (largest power of two not above amax, divided by the
    largest power of two the element type represents) on random blocks, and
    saturation at the largest normal;
  * the FP6 bit packing round-trips and puts element i at bits 6i.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from golden_io import lines
from oracle import elements as el

FP8_TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def test_family_table_widths():
    rows = [ln.split() for ln in lines("mx_family.txt")]
    for fmt, et, bits, block, scale in rows:
        assert int(block) == 32 and scale == "E8M0"
        name = et.lower()
        if name == "e2m1":
            continue
        e, m = int(name[1]), int(name[3])
        assert 1 + e + m == int(bits) == el.elem_bits(name)
        assert el.block_bits(name) == 32 * int(bits) + 8
        assert (fmt == "MXFP8") == (int(bits) == 8)


@pytest.mark.parametrize("elem", ["e4m3", "e5m2"])
def test_fp8_decode_matches_torch_on_every_code(elem):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(FP8_TORCH[elem]).float().numpy().astype(np.float64)
    got = el.decode(codes, elem)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def _probe_values(elem):
    g = el.grid(elem)
    pts = set(g.tolist())
    pts.update(((g[:-1] + g[1:]) / 2).tolist())
    out = set()
    for p in pts:
        f = np.float32(p)
        for d in (-2, -1, 0, 1, 2):
            v = f
            for _ in range(abs(d)):
                v = np.nextafter(v, np.float32(np.inf) if d > 0 else np.float32(0))
            out.add(float(v))
    return np.array(sorted(v for v in out if v <= g[-1]), dtype=np.float32)


@pytest.mark.parametrize("elem", ["e4m3", "e5m2"])
def test_fp8_rne_matches_torch(elem):
    """Grid points, midpoints (ties) and +-2 ulps around them, both signs, and
    random values below the largest normal: the oracle's code equals torch's
    float32 -> float8 cast (round to nearest even)."""
    rng = np.random.default_rng(1)
    top = el.max_normal(elem)
    v = np.concatenate([_probe_values(elem),
                        (rng.uniform(-1, 1, 20000) * top).astype(np.float32),
                        np.exp(rng.uniform(-25, math.log(top), 20000)).astype(np.float32)])
    v = np.concatenate([v, -v])
    got = el.round_elem(v, elem, "rne")
    ref = torch.from_numpy(v).to(FP8_TORCH[elem]).view(torch.uint8).numpy().astype(np.int64)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("elem", ["e2m3", "e3m2"])
def test_fp6_rne_bruteforce(elem):
    """Nearest grid value by exhaustive distance, ties to the even code,
    saturating above the largest normal; the grid's end points are the
    definitions' closed forms."""
    g = el.grid(elem)
    e, m, top = el.ELEMS[elem]
    bias = (1 << (e - 1)) - 1
    assert g[-1] == (2 - 2.0 ** -m) * 2.0 ** ((1 << e) - 1 - bias)
    assert g[1] == 2.0 ** (1 - bias - m)
    v = np.concatenate([_probe_values(elem), np.float32([g[-1] * 1.01, 1e9])])
    got = el.round_elem(v, elem, "rne")
    for x, c in zip(v, got):
        d = np.abs(g - float(x))
        best = min(range(len(g)), key=lambda i: (d[i], i % 2))
        assert c == best, (elem, float(x), c, best)
    assert np.array_equal(el.round_elem(-v, elem, "rne"), got | (1 << (e + m)))


@pytest.mark.parametrize("elem", list(el.ELEMS))
def test_scale_rule_and_saturation(elem):
    """X = (largest power of two <= amax) / (largest power of two of the type);
    every scaled element is at most the largest normal after saturation, and
    a value just below amax keeps its sign and code magnitude <= largest."""
    rng = np.random.default_rng(3)
    x = (rng.standard_t(3, (16, 32 * 4)) * np.exp(rng.uniform(-8, 8, (16, 1)))).astype(np.float32)
    codes, scales = oracle.quantize(x, elem=elem)
    g = el.grid(elem)
    p2 = 2.0 ** math.floor(math.log2(g[-1]))        # largest power of two of the type, by brute force
    assert p2 == 2.0 ** el.emax(elem)
    for r in range(16):
        for b in range(4):
            amax = float(np.abs(x[r, b * 32:(b + 1) * 32]).max())
            X = 2.0 ** math.floor(math.log2(amax)) / p2
            assert float(oracle.e8m0_decode(scales[r, b])) == X
    deq = oracle.dequantize(codes, scales, elem=elem).astype(np.float64)
    sc = np.repeat(oracle.e8m0_decode(scales), 32, axis=1)
    assert np.all(np.abs(deq) <= g[-1] * sc)
    assert np.all(np.sign(deq[deq != 0]) == np.sign(x[deq != 0]))


def test_fp6_packing():
    rng = np.random.default_rng(4)
    c = rng.integers(0, 64, (3, 64))
    p = el.pack(c, "e2m3")
    assert p.shape == (3, 48)
    assert np.array_equal(el.unpack(p, "e2m3", 64), c)
    one = np.zeros((1, 32), dtype=np.int64)
    one[0, 1] = 0x3F                        # element 1 -> bits 6..11
    q = el.pack(one, "e3m2")[0]
    assert q[0] == 0xC0 and q[1] == 0x0F and not q[2:].any()


@pytest.mark.parametrize("elem", list(el.ELEMS))
def test_quantize_error_bound(elem):
    """|x - deq(q(x))| <= half a grid step at |x| (no element of these blocks
    exceeds the largest normal after scaling: amax/X < 2 * 2^emax, and the
    clip band above the largest normal is counted separately)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    codes, scales = oracle.quantize(x, elem=elem)
    deq = oracle.dequantize(codes, scales, elem=elem).astype(np.float64)
    sc = np.repeat(oracle.e8m0_decode(scales), 32, axis=1)
    g = el.grid(elem)
    v = np.abs(x) / sc
    i = np.clip(np.searchsorted(g, v, side="right") - 1, 0, len(g) - 2)
    step = g[i + 1] - g[i]
    err = np.abs(x - deq) / sc
    clip = v > g[-1]
    assert np.all(err[~clip] <= step[~clip] / 2 + 1e-12)
    assert np.allclose(err[clip], v[clip] - g[-1])


def test_gemm_ref_mixed_types_bruteforce():
    """A block dot product of an FP8 row with an FP6 row equals the exact
    rational sum of the decoded products."""
    from fractions import Fraction
    rng = np.random.default_rng(6)
    a = rng.integers(0, 0x7E, (1, 32)) | (rng.integers(0, 2, (1, 32)) << 7)
    b = rng.integers(0, 64, (1, 32))
    ac, bc = el.pack(a, "e4m3"), el.pack(b, "e3m2")
    ref, _ = oracle.gemm_ref(ac, np.array([[125]], np.uint8), bc, np.array([[130]], np.uint8),
                             a_elem="e4m3", b_elem="e3m2")
    exact = sum(Fraction(float(p)) * Fraction(float(q))
                for p, q in zip(el.decode(a[0], "e4m3"), el.decode(b[0], "e3m2"))) * Fraction(2) ** 1
    assert ref[0, 0] == float(exact)


# ---------------------------------------------------------------- pins written from the definitions alone
def _fp6_value_exact(code, e, m):
    """Value of a FP6 code as an exact fraction, from the floating-point
    definition: sign bit, e exponent bits with bias 2^(e-1) - 1, m mantissa
    bits; exponent field 0 is subnormal, (f / 2^m) * 2^(1 - bias)."""
    from fractions import Fraction
    bias = (1 << (e - 1)) - 1
    sign = -1 if (code >> (e + m)) & 1 else 1
    E = (code >> m) & ((1 << e) - 1)
    f = code & ((1 << m) - 1)
    if E == 0:
        mag = Fraction(f, 1 << m) * Fraction(2) ** (1 - bias)
    else:
        mag = (1 + Fraction(f, 1 << m)) * Fraction(2) ** (E - bias)
    return sign * mag


@pytest.mark.parametrize("elem", ["e2m3", "e3m2"])
def test_fp6_decode_every_code_against_exact_enumeration(elem):
    """All 64 codes of each FP6 type decode to the exact value the
    definition gives (OCP MX v1.0 element definitions, read for the types
    "MXFP4", AI Wiki, §Place in the MX family names); -0 keeps its sign."""
    e, m, _ = el.ELEMS[elem]
    got = el.decode(np.arange(64), elem)
    for c in range(64):
        want = _fp6_value_exact(c, e, m)
        assert got[c] == float(want), (elem, c, got[c], want)
        if want == 0:
            assert math.copysign(1.0, got[c]) == (-1.0 if c >> (e + m) else 1.0)
    # the grid is strictly increasing and has 32 finite magnitudes
    g = el.grid(elem)
    assert len(g) == 32 and np.all(np.diff(g) > 0)


def _sr_probe_points(elem, rng, n=40):
    """Random float32 values strictly between neighbouring grid points
    (below the largest normal), with their exact neighbours and fraction."""
    from fractions import Fraction
    g = el.grid(elem)
    out = []
    for _ in range(n):
        i = int(rng.integers(0, len(g) - 1))
        lo, hi = g[i], g[i + 1]
        v = np.float32(lo + (hi - lo) * rng.uniform(0.01, 0.99))
        if not lo < float(v) < hi:
            continue
        f = (Fraction(float(v)) - Fraction(lo)) / (Fraction(hi) - Fraction(lo))
        out.append((v, i, f))
    return out


@pytest.mark.parametrize("elem", list(el.ELEMS))
def test_sr_threshold_bruteforce(elem):
    """Stochastic rounding with 16-bit draws r: up iff r < f * 2^16, f the
    exact fraction of the way from the lower to the upper neighbour.  Checked
    at the draws T - 1, T, T + 1 around T = floor(f * 2^16), for fractions with
    and without an exact 16-bit representation (an integer f * 2^16 rounds
    down at r = T, any other rounds up at r = T)."""
    from fractions import Fraction
    rng = np.random.default_rng(31)
    pts = _sr_probe_points(elem, rng)
    g = el.grid(elem)
    # fractions that are exact multiples of 2^-16: midpoints and quarter points
    for i in range(0, len(g) - 1, 3):
        for q in (Fraction(1, 2), Fraction(1, 4), Fraction(3, 4)):
            v = Fraction(g[i]) + q * (Fraction(g[i + 1]) - Fraction(g[i]))
            if np.float32(float(v)) == float(v):
                pts.append((np.float32(float(v)), i, q))
    assert len(pts) > 30
    e, m, _ = el.ELEMS[elem]
    for v, i, f in pts:
        t = math.floor(f * 65536)
        exact = f * 65536 == t
        for r in (t - 1, t, t + 1):
            if not 0 <= r < 65536:
                continue
            code = int(el.round_elem(np.float32([v]), elem, "sr", np.uint32([r]))[0])
            up = r < f * 65536
            assert code == i + int(up), (elem, float(v), r, code, i)
            if r == t:
                assert up == (not exact)
            neg = int(el.round_elem(np.float32([-v]), elem, "sr", np.uint32([r]))[0])
            assert neg == code | (1 << (e + m))


@pytest.mark.parametrize("elem", list(el.ELEMS))
def test_sr_unbiased_with_binomial_variance(elem):
    """Over n uniform 16-bit draws the mean of the stochastically rounded
    value is v within 5 sigma / sqrt(n) plus the 2^-16 step term, sigma^2 =
    (v - lo)(hi - v) in closed form, and the variance is that binomial one."""
    rng = np.random.default_rng(32)
    n = 100_000
    g = el.grid(elem)
    for v, i, f in _sr_probe_points(elem, rng, n=6):
        lo, hi = float(g[i]), float(g[i + 1])
        r = rng.integers(0, 65536, n).astype(np.uint32)
        got = el.decode(el.round_elem(np.full(n, v, np.float32), elem, "sr", r), elem)
        assert set(np.unique(got)) <= {lo, hi}
        x = float(v)
        sigma = math.sqrt((x - lo) * (hi - x))
        tol = 5 * sigma / math.sqrt(n) + (hi - lo) * 2.0 ** -16
        assert abs(got.mean() - x) <= tol, (elem, x)
        assert abs(got.var() - sigma ** 2) <= 0.05 * sigma ** 2 + 1e-12 * hi * hi


def _round_up_exponent_bruteforce(amax, top):
    """Smallest integer e in [-127, 127] with amax <= top * 2^e, by search
    (top * 2^e is exact in binary floating point)."""
    for e in range(-127, 128):
        if amax <= top * 2.0 ** e:
            return e
    return 127


@pytest.mark.parametrize("elem,top", [("e4m3", 448.0), ("e5m2", 57344.0), ("e2m3", 7.5), ("e3m2", 28.0)])
def test_round_up_scale_bruteforce_per_type(elem, top):
    """Round-up scale rule for the other element types: the smallest power of
    two 2^e with amax <= (largest normal) * 2^e ("MXFP4", AI Wiki, §Clipping
    in the reference algorithm, with the type's largest normal in place of 6),
    by exhaustive search, at random magnitudes and at top * 2^k and its float32
    neighbours for every k in range; codes then never saturate: every scaled
    element is at most top and rounds to the nearest grid value."""
    assert el.max_normal(elem) == top             # the definitions' largest normal
    rng = np.random.default_rng(33)
    mags = [float(np.float32(v)) for v in np.ldexp(rng.uniform(1.0, 2.0, 1500), rng.integers(-140, 120, 1500))]
    for k in range(-150, 128):
        if top * 2.0 ** k >= float(np.finfo(np.float32).max):
            break
        b = np.float32(top * 2.0 ** k)
        if b == 0:
            continue
        mags += [float(b), float(np.nextafter(b, np.float32(np.inf))), float(np.nextafter(b, np.float32(0)))]
    mags = [x for x in mags if 0 < x < float(np.finfo(np.float32).max)]
    g = el.grid(elem)
    x = np.zeros((len(mags), 32), dtype=np.float32)
    x[:, 3] = mags
    x[:, 7] = np.float32(mags) * np.float32(0.3)
    codes, scales = oracle.quantize(x, elem=elem, scale_mode="round_up")
    deq = oracle.dequantize(codes, scales, elem=elem)
    for r, amax in enumerate(mags):
        e = _round_up_exponent_bruteforce(float(np.float32(amax)), top)
        assert int(scales[r, 0]) == e + 127, (elem, amax)
        if e > -127:
            v = float(np.float32(amax)) / 2.0 ** e
            assert top / 2 < v <= top
            # nearest grid value (no clipping); ties cannot move it above top
            assert abs(abs(float(deq[r, 3])) / 2.0 ** e - v) <= np.max(np.diff(g)) / 2
            assert abs(float(deq[r, 3])) <= top * 2.0 ** e
