"""GPU parity of the MXFP8 / MXFP6 element types against the oracle.

Quantizer and dequantizer: codes, scales and decoded values bit-exact (the
quantizer rounds in software on the GPU, so there is no allowance).  GEMM: the
oracle's float64 reference of the oracle's own operands, within
1e-5 * sum |a_k b_k| plus the scaled MFMA's internal-precision allowance for
FP8/FP6 operands (gpu_util.mx_group_bound, measured by the probe tests).
"""
import zlib

import numpy as np
import pytest
import torch

import mxfp4_microscaling_quantization_mx_amd as mx
import oracle
from gpu_util import banner, bf16_half_ulp, codes_equal, host, mx_group_bound, need_gpu, to_dev
from oracle import elements as el

pytestmark = pytest.mark.gpu

ELEMS = ["e4m3", "e5m2", "e2m3", "e3m2"]


def _case_id(elem, axis, rounding, rht):
    return f"{elem}-{axis}-{rounding}-{'rht' if rht else 'plain'}"


CASES = [(e, a, r, h) for e in ELEMS for a in ("last", "dim0") for r in ("rne", "sr", "sr8") for h in (False, True)]


@pytest.mark.parametrize("elem,axis,rounding,rht", CASES, ids=[_case_id(*c) for c in CASES])
def test_quantize_elements(elem, axis, rounding, rht):
    """Every element type along both axes, RNE and stochastic rounding, with and
    without the transform, on ragged bf16 shapes: bit-exact."""
    need_gpu()
    R, C = (72, 416) if axis == "last" else (224, 88)
    rng = np.random.default_rng(zlib.crc32(_case_id(elem, axis, rounding, rht).encode()))
    x = (rng.standard_t(3, (R, C)) * np.exp(rng.uniform(-6, 6, (R, 1)))).astype(np.float32)
    xt = torch.from_numpy(x).to(torch.bfloat16)
    kw = dict(axis=axis, rounding=rounding, rht_mask=0x5A5A1234 if rht else None, seed=0xABCDEF12345, offset=3)
    banner(f"quantize {_case_id(elem, axis, rounding, rht)} R={R} C={C}")
    q = mx.quantize(xt.cuda(), elem=elem, **kw)
    oc, os_ = oracle.quantize(xt.float().numpy(), elem=elem, **kw)
    codes_equal(host(q.scales), os_, "scales")
    codes_equal(host(q.codes), oc, "codes")


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("axis", ["last", "dim0"])
@pytest.mark.parametrize("rounding,rht", [("rne", False), ("sr", True), ("sr8", False)])
def test_quantize_elements_2d(elem, axis, rounding, rht):
    """32x32 tiles (one scale per tile) for every element type, along the
    last dim (LDS tile kernel) and dim 0 (column kernel), ragged in K."""
    need_gpu()
    R, C = (96, 352) if axis == "last" else (224, 96)
    rng = np.random.default_rng(zlib.crc32(f"2d{elem}{axis}{rounding}".encode()))
    x = (rng.standard_t(3, (R, C)) * np.exp(rng.uniform(-6, 6, (R, 1)))).astype(np.float32)
    kw = dict(axis=axis, block="2d", rounding=rounding, rht_mask=0x13579BDF if rht else None, seed=21, offset=2)
    banner(f"quantize 2d {elem} {axis} {rounding} rht={rht}")
    q = mx.quantize(to_dev(x), elem=elem, **kw)
    oc, os_ = oracle.quantize(x, elem=elem, **kw)
    codes_equal(host(q.scales), os_, "scales")
    codes_equal(host(q.codes), oc, "codes")


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("scale_mode", ["round_up", "prescale_3_4"])
def test_quantize_elements_scale_modes_f32(elem, scale_mode):
    need_gpu()
    rng = np.random.default_rng(7 + ELEMS.index(elem))
    x = (rng.standard_normal((40, 160)) * np.exp(rng.uniform(-9, 9, (40, 1)))).astype(np.float32)
    banner(f"quantize {elem} {scale_mode} f32")
    q = mx.quantize(to_dev(x), elem=elem, scale_mode=scale_mode, rounding="sr", seed=5)
    oc, os_ = oracle.quantize(x, elem=elem, scale_mode=scale_mode, rounding="sr", seed=5)
    codes_equal(host(q.scales), os_, "scales")
    codes_equal(host(q.codes), oc, "codes")


def _adversarial(elem):
    """Blocks whose scaled values sit on grid points, midpoints (ties) and
    +-1 ulp around them, in the clip band above the largest normal, in the
    subnormal range, plus zero, NaN and Inf blocks and extreme magnitudes."""
    g = el.grid(elem)
    top = g[-1]
    p2 = 2.0 ** el.emax(elem)
    vals = [float(v) for v in g] + [float((a + b) / 2) for a, b in zip(g[:-1], g[1:])]
    vals += [float(np.nextafter(np.float32(v), np.float32(np.inf))) for v in vals[:40]]
    vals += [top * 1.01, top * 1.1, 2 * p2 * 0.999, -top, -g[1] / 2]
    rows = []
    vals = np.array(vals, dtype=np.float64)
    for i in range(0, len(vals), 31):
        chunk = list(vals[i:i + 31])
        chunk = (chunk + [0.0] * 31)[:31] + [p2]            # pins the scale byte at the type's 2^emax
        rows.append(chunk)
    rows = [r for r in rows]
    for scale in (2.0 ** -100, 2.0 ** 60):
        rows.append([v * scale for v in rows[0]])
    rows.append([0.0] * 32)
    r = [1.0] * 32
    r[5] = np.nan
    rows.append(r)
    r = [1.0] * 32
    r[9] = np.inf
    rows.append(r)
    rows.append([3e38] * 16 + [1e-39] * 16)
    x = np.array(rows, dtype=np.float32)
    if len(x) % 2:
        x = np.concatenate([x, np.zeros((1, 32), np.float32)])
    return x.reshape(-1, 64)


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_quantize_elements_adversarial(elem, rounding):
    need_gpu()
    x = _adversarial(elem)
    banner(f"quantize {elem} adversarial {rounding}")
    q = mx.quantize(to_dev(x), elem=elem, rounding=rounding, seed=77)
    oc, os_ = oracle.quantize(x, elem=elem, rounding=rounding, seed=77)
    codes_equal(host(q.scales), os_, "scales")
    codes_equal(host(q.codes), oc, "codes")


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("block", ["1d", "2d"])
def test_dequantize_elements(elem, block):
    """Random code bytes (NaN and Inf codes included) and scales (the NaN
    scale included), decoded bit-exactly to float32 and to bf16 (RNE)."""
    need_gpu()
    rng = np.random.default_rng(11 + ELEMS.index(elem) + 4 * (block == "2d"))
    R, K = 64, 192
    cb = K * el.elem_bits(elem) // 8
    codes = rng.integers(0, 256, (R, cb), dtype=np.uint8)
    srows = R // 32 if block == "2d" else R
    scales = rng.integers(100, 150, (srows, K // 32), dtype=np.uint8)
    scales[0, 1] = 0xFF
    q = mx.empty_mx(R, K, block, elem=elem)
    q.codes.copy_(to_dev(codes))
    q.scales.copy_(to_dev(scales))
    banner(f"dequantize {elem} {block}")
    got = host(mx.dequantize(q, torch.float32))
    ref = oracle.dequantize(codes, scales, block, elem=elem)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    gb = host(mx.dequantize(q, torch.bfloat16).view(torch.int16)).astype(np.int64) & 0xFFFF
    rb = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64) & 0xFFFF
    assert np.array_equal(gb[ok], rb[ok])



@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("block", ["1d", "2d"])
def test_dequantize_elements_inverse_rht(elem, block):
    """The decode followed by the inverse 32-point transform (a lane per block,
    all five butterfly stages in registers) on random code bytes and scales
    of every element type: float32 bit-exact against the oracle's transform in
    its fixed stage order (NaN wherever the oracle has NaN), bf16 its RNE
    rounding."""
    need_gpu()
    rng = np.random.default_rng(71 + ELEMS.index(elem) + 4 * (block == "2d"))
    R, K = 96, 224
    cb = K * el.elem_bits(elem) // 8
    codes = rng.integers(0, 256, (R, cb), dtype=np.uint8)
    srows = R // 32 if block == "2d" else R
    scales = rng.integers(110, 140, (srows, K // 32), dtype=np.uint8)
    scales[-1, 2] = 0xFF
    mask = 0x9E3779B9
    q = mx.empty_mx(R, K, block, elem=elem)
    q.codes.copy_(to_dev(codes))
    q.scales.copy_(to_dev(scales))
    banner(f"dequantize {elem} {block} inverse rht")
    got = host(mx.dequantize(q, torch.float32, inverse_rht_mask=mask))
    ref = oracle.dequantize(codes, scales, block, inverse_rht_mask=mask, elem=elem).astype(np.float32)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    gb = host(mx.dequantize(q, torch.bfloat16, inverse_rht_mask=mask).view(torch.int16)).astype(np.int64) & 0xFFFF
    rb = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64) & 0xFFFF
    assert np.array_equal(gb[ok], rb[ok])

def _finite_codes(rng, elem, shape):
    if elem == "e2m1":
        return rng.integers(0, 16, size=shape)
    e, m, top = el.ELEMS[elem]
    return rng.integers(0, top + 1, size=shape) | (rng.integers(0, 2, size=shape) << (e + m))


def _pack(codes, elem):
    return oracle.pack_nibbles(codes) if elem == "e2m1" else el.pack(codes, elem)


def _operand(rng, rows, K, elem, block="1d"):
    codes = _pack(_finite_codes(rng, elem, (rows, K)), elem)
    srows = rows // 32 if block == "2d" else rows
    scales = rng.integers(115, 140, (srows, K // 32), dtype=np.uint8)
    q = mx.empty_mx(rows, K, block, elem=elem)
    q.codes.copy_(to_dev(codes))
    q.scales.copy_(to_dev(scales))
    return q, codes, scales


GEMM_CASES = [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e2m3", "e2m3"), ("e3m2", "e3m2"), ("e4m3", "e2m1"),
              ("e2m1", "e5m2"), ("e2m3", "e4m3"), ("e3m2", "e2m1"), ("e4m3", "e3m2")]


@pytest.mark.parametrize("fa,fb", GEMM_CASES)
@pytest.mark.parametrize("M,N,K,b_block,out", [(200, 136, 416, "1d", torch.float32),
                                               (96, 160, 96, "2d", torch.bfloat16),
                                               (300, 544, 224, "2d", torch.bfloat16),
                                               (520, 288, 800, "1d", torch.float32)])
def test_gemm_elements(fa, fb, M, N, K, b_block, out):
    """Mixed and uniform element types on ragged shapes (rows, columns and K
    not multiples of the tile: the 128x128 kernel below 256 rows or columns,
    the 256x256 one above), 1-D and 2-D B scales, float32 and bf16 outputs."""
    need_gpu()
    rng = np.random.default_rng(zlib.crc32(f"{fa}{fb}{M}{N}{K}".encode()))
    qa, ac, as_ = _operand(rng, M, K, fa)
    qb, bc, bs = _operand(rng, N, K, fb, b_block)
    banner(f"gemm {fa} x {fb} M={M} N={N} K={K} {b_block} {out}")
    c = host(mx.gemm(qa, qb, out).float()).astype(np.float64)
    ref, bound = oracle.gemm_ref(ac, as_, bc, bs, "1d", b_block, a_elem=fa, b_elem=fb)
    av = oracle.gemm.dequant_f64(ac, as_, fa)
    bv = oracle.gemm.dequant_f64(bc, bs, fb, b_block)
    gb = mx_group_bound(av, bv)
    tol = 1e-5 * bound + gb
    if out == torch.bfloat16:
        tol = tol + bf16_half_ulp(np.maximum(np.abs(c), np.abs(ref)))
    err = np.abs(c - ref)
    assert np.all(err <= tol), float(np.max(err / tol))
    if out == torch.float32 and fa + fb != "e2m1e2m1":
        # the error beyond the float32 accumulation bound, as a fraction of
        # the instruction's alignment allowance: the truncation is real (the
        # allowance is used) but stays well inside it; on these seeded cases
        # (deterministic results) it reaches 0.43 (e2m3 x e4m3, K = 800)
        excess = np.maximum(err - 1e-5 * bound, 0.0)
        ratio = float(np.max(excess / np.maximum(gb, 1e-300)))
        print(f"[excess/allowance] {fa} x {fb} M={M} N={N} K={K}: {ratio:.4f}")
        assert ratio <= 0.5, ratio


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e2m3", "e3m2")])
@pytest.mark.parametrize("M,N", [(200, 136), (300, 544)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_gemm_elements_guard(fa, fb, M, N, out):
    """C inside a larger buffer filled with a marker, rows and columns ragged
    against both tile sizes: the kernel's bounds-checked buffer stores write
    C and nothing else."""
    need_gpu()
    K = 224
    rng = np.random.default_rng(zlib.crc32(f"guard{fa}{fb}{M}{N}".encode()))
    qa, ac, as_ = _operand(rng, M, K, fa)
    qb, bc, bs = _operand(rng, N, K, fb)
    buf = torch.full((M + 37, N + 21), 7.0, dtype=out, device="cuda")
    banner(f"gemm guard {fa} x {fb} M={M} N={N} {out}")
    mx.gemm(qa, qb, out=buf[:M, :N])
    got = host(buf.float()).astype(np.float64)
    assert np.all(got[M:] == 7.0) and np.all(got[:, N:] == 7.0), "wrote outside C"
    ref, bound = oracle.gemm_ref(ac, as_, bc, bs, a_elem=fa, b_elem=fb)
    tol = 1e-5 * bound + mx_group_bound(oracle.gemm.dequant_f64(ac, as_, fa), oracle.gemm.dequant_f64(bc, bs, fb))
    if out == torch.bfloat16:
        tol = tol + bf16_half_ulp(np.maximum(np.abs(got[:M, :N]), np.abs(ref)))
    assert np.all(np.abs(got[:M, :N] - ref) <= tol)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e2m3", "e2m3"), ("e5m2", "e3m2")])
def test_gemm_mxfp8_end_to_end(fa, fb):
    """MXFP8 / MXFP6 activations times weights quantized on the GPU (the
    weights along dim 0), 2048 x 1024 x 2880, against the oracle on sampled
    rows and columns."""
    need_gpu()
    rng = np.random.default_rng(12)
    x = rng.standard_normal((2048, 2880)).astype(np.float32)
    w = (rng.standard_normal((2880, 1024)) * 0.02).astype(np.float32)
    xt, wt = torch.from_numpy(x).to(torch.bfloat16), torch.from_numpy(w).to(torch.bfloat16)
    banner(f"gemm {fa} x {fb} end to end")
    qx = mx.quantize(xt.cuda(), elem=fa)
    qw = mx.quantize(wt.cuda(), axis="dim0", elem=fb)
    y = host(mx.gemm(qx, qw, torch.float32)).astype(np.float64)
    rows = np.sort(rng.choice(2048, 32, replace=False))
    cols = np.sort(rng.choice(1024, 32, replace=False))
    xc, xs = oracle.quantize(xt.float().numpy()[rows], elem=fa)
    wc, ws = oracle.quantize(wt.float().numpy()[:, cols], axis="dim0", elem=fb)
    ref, bound = oracle.gemm_ref(xc, xs, wc, ws, a_elem=fa, b_elem=fb)
    tol = 1e-5 * bound + mx_group_bound(oracle.gemm.dequant_f64(xc, xs, fa),
                                        oracle.gemm.dequant_f64(wc, ws, fb))
    assert np.all(np.abs(y[np.ix_(rows, cols)] - ref) <= tol)


# (exponent-field range, E, M) of "narrow" codes: normal values in [1, 16)
_NARROW = {"e4m3": (7, 10, 4, 3), "e5m2": (15, 18, 5, 2), "e2m3": (1, 3, 2, 3), "e3m2": (3, 6, 3, 2)}


def _narrow_codes(rng, elem, shape):
    """Random signs and mantissas over four binades of normals, so that the
    products of one 64-deep MFMA step lie within 2^10 of each other, inside
    the instruction's alignment window: the float32 bound alone applies."""
    lo, hi, E, M = _NARROW[elem]
    e = rng.integers(lo, hi + 1, size=shape)
    m = rng.integers(0, 1 << M, size=shape)
    sgn = rng.integers(0, 2, size=shape)
    return _pack((sgn << (E + M)) | (e << M) | m, elem)


@pytest.mark.parametrize("fa,fb,out", [("e4m3", "e4m3", torch.bfloat16), ("e2m3", "e3m2", torch.float32),
                                       ("e5m2", "e2m3", torch.bfloat16)])
def test_gemm_elements_more_tiles_than_cus(fa, fb, out):
    """4352 x 4160 x 416: 17 x 17 tiles of 256 (the last column tile 64 wide),
    more than there are CUs, so workgroups of the persistent direct-to-LDS
    kernel run a second tile (its first stage loaded during the first tile's
    last stage and epilogue); K = 416 is 3.25 stages and, for FP6, ends half-way
    through a 16-byte chunk.  Every output against the oracle."""
    need_gpu()
    M, N, K = 4352, 4160, 416
    rng = np.random.default_rng(zlib.crc32(f"many{fa}{fb}".encode()))
    ac, bc = _narrow_codes(rng, fa, (M, K)), _narrow_codes(rng, fb, (N, K))
    as_ = np.full((M, K // 32), 127, dtype=np.uint8)
    bs = rng.integers(125, 130, (N, K // 32), dtype=np.uint8)
    as_[:, 1::2] = 126
    qa, qb = mx.empty_mx(M, K, elem=fa), mx.empty_mx(N, K, elem=fb)
    qa.codes.copy_(to_dev(ac)); qa.scales.copy_(to_dev(as_))
    qb.codes.copy_(to_dev(bc)); qb.scales.copy_(to_dev(bs))
    banner(f"gemm {fa} x {fb} {M}x{N}x{K} {out}")
    c = host(mx.gemm(qa, qb, out).float()).astype(np.float64)
    ref, bound = oracle.gemm_ref(ac, as_, bc, bs, a_elem=fa, b_elem=fb)
    tol = 1e-5 * bound
    if out == torch.bfloat16:
        tol = tol + bf16_half_ulp(np.maximum(np.abs(c), np.abs(ref)))
    err = np.abs(c - ref)
    assert np.all(err <= tol), float(np.max(err / tol))


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e2m3", "e3m2"), ("e5m2", "e2m1")])
@pytest.mark.parametrize("N", [160, 288])
def test_grouped_gemm_elements(fa, fb, N):
    """MoE grouped GEMM with MXFP8/MXFP6 operands: empty experts, a one-row
    expert, experts straddling row tiles, rows past the last offset left
    untouched; B stacked per expert with 2-D scales."""
    need_gpu()
    rng = np.random.default_rng(zlib.crc32(f"g{fa}{fb}{N}".encode()))
    offsets = np.array([0, 0, 1, 300, 300, 557, 700], dtype=np.int32)
    E, K, M = len(offsets) - 1, 160, 720
    ac = _pack(_finite_codes(rng, fa, (M, K)), fa)
    as_ = rng.integers(118, 136, (M, K // 32), dtype=np.uint8)
    bc = np.stack([_pack(_finite_codes(rng, fb, (N, K)), fb) for _ in range(E)])
    bs = rng.integers(118, 136, (E, N // 32, K // 32), dtype=np.uint8)
    qa = mx.empty_mx(M, K, elem=fa)
    qa.codes.copy_(to_dev(ac))
    qa.scales.copy_(to_dev(as_))
    qb = mx.empty_mx(N, K, "2d", experts=E, elem=fb)
    qb.codes.copy_(to_dev(bc))
    qb.scales.copy_(to_dev(bs))
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    banner(f"grouped gemm {fa} x {fb} N={N}")
    mx.grouped_gemm(qa, torch.from_numpy(offsets).cuda(), qb, out=y)
    got = host(y).astype(np.float64)
    ref, bound = oracle.grouped_gemm_ref(ac, as_, offsets, bc, bs, "1d", "2d", rows=np.arange(700),
                                         a_elem=fa, b_elem=fb)
    av = oracle.gemm.dequant_f64(ac[:700], as_[:700], fa)
    tol = 1e-5 * bound
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            bv = oracle.gemm.dequant_f64(bc[e], bs[e], fb, "2d")
            tol[lo:hi] += mx_group_bound(av[lo:hi], bv)
    assert np.all(np.abs(got[:700] - ref) <= tol)
    assert np.all(got[700:] == 7.0)


@pytest.mark.parametrize("fa,fb,b_block", [("e4m3", "e4m3", "2d"), ("e2m3", "e3m2", "1d"), ("e5m2", "e2m3", "2d")])
def test_grouped_gemm_elements_more_tiles_than_cus(fa, fb, b_block):
    """Grouped MXFP8 / MXFP6 GEMM with skewed experts (an empty one, a
    one-row one, experts straddling row tiles) over 8192 routed rows, N = 2336
    (the last column tile 32 wide), K = 416: about 360 tiles, more than there
    are CUs, so the persistent direct-to-LDS kernel runs second tiles; bf16
    output; every routed row against the oracle, rows past the last offset
    untouched."""
    need_gpu()
    rng = np.random.default_rng(zlib.crc32(f"gm{fa}{fb}{b_block}".encode()))
    offsets = np.array([0, 700, 700, 701, 2900, 3000, 5500, 8000, 8100], dtype=np.int32)
    E, K, N, M = len(offsets) - 1, 416, 2336, 8192
    ac = _narrow_codes(rng, fa, (M, K))
    as_ = rng.integers(126, 129, (M, K // 32), dtype=np.uint8)
    bc = np.stack([_narrow_codes(rng, fb, (N, K)) for _ in range(E)])
    srows = N // 32 if b_block == "2d" else N
    bs = rng.integers(125, 129, (E, srows, K // 32), dtype=np.uint8)
    qa = mx.empty_mx(M, K, elem=fa)
    qa.codes.copy_(to_dev(ac)); qa.scales.copy_(to_dev(as_))
    qb = mx.empty_mx(N, K, b_block, experts=E, elem=fb)
    qb.codes.copy_(to_dev(bc)); qb.scales.copy_(to_dev(bs))
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    banner(f"grouped gemm {fa} x {fb} {b_block} {M}x{N}x{K} E={E}")
    mx.grouped_gemm(qa, torch.from_numpy(offsets).cuda(), qb, out=y)
    got = host(y.float()).astype(np.float64)
    last = int(offsets[-1])
    ref, bound = oracle.grouped_gemm_ref(ac, as_, offsets, bc, bs, "1d", b_block, rows=np.arange(last),
                                         a_elem=fa, b_elem=fb)
    tol = 1e-5 * bound + bf16_half_ulp(np.maximum(np.abs(got[:last]), np.abs(ref)))
    assert np.all(np.abs(got[:last] - ref) <= tol)
    assert np.all(got[last:] == 7.0)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e2m3", "e3m2")])
def test_gemm_elements_zero_k(fa, fb):
    """K = 0 on the direct-to-LDS kernels (dense 300 x 544 and grouped with
    N = 288): every output is zero (no stage is loaded or multiplied), rows
    past the last expert offset untouched."""
    need_gpu()
    banner(f"gemm K=0 {fa} x {fb}")
    y = torch.full((300, 544), 7.0, dtype=torch.float32, device="cuda")
    mx.gemm(mx.empty_mx(300, 0, elem=fa), mx.empty_mx(544, 0, elem=fb), out=y)
    assert np.all(host(y) == 0.0)
    offsets = torch.tensor([0, 0, 260, 290], dtype=torch.int32, device="cuda")
    g = torch.full((300, 288), 7.0, dtype=torch.bfloat16, device="cuda")
    mx.grouped_gemm(mx.empty_mx(300, 0, elem=fa), offsets, mx.empty_mx(288, 0, "2d", experts=3, elem=fb), out=g)
    gh = host(g.float())
    assert np.all(gh[:290] == 0.0) and np.all(gh[290:] == 7.0)
