"""In-bounds checks of the gfx950 builtins the library relies on.

* Scaled FP4 MFMA operand / scale / result lane layouts, checked against a
  NumPy model of C = sum_k (A[i,k] X_A[i,k/32]) (B[j,k] X_B[j,k/32]).
* The hardware packed FP4 conversion (scale 1.0) against the library's
  software RNE over every float32 input: the quantizer uses the hardware
  instruction for RNE, which is only valid while the two agree everywhere.
* The hardware stochastic-rounding conversion, as the library drives it,
  against the library's software SR rule for every float32 |x| < 8 at the
  draws around each rounding threshold.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_util import banner, mx_group_bound, need_gpu, probe_lib, save_npz

pytestmark = pytest.mark.gpu


def _lane_regs(mat_codes, rows_per_tile, kgroups):
    """Per-lane 8 x int32 operand registers for an FP4 MFMA operand.

    mat_codes: [rows_per_tile, 32*kgroups] codes.  Lane l holds row
    l % rows_per_tile and K-elements [32*g, 32*g+32) with g = l // rows_per_tile,
    two codes per byte (even element low nibble) in the first 4 registers."""
    regs = np.zeros((64, 8), dtype=np.uint32)
    for l in range(64):
        r, g = l % rows_per_tile, l // rows_per_tile
        seg = mat_codes[r, 32 * g:32 * g + 32].astype(np.uint32)
        by = seg[0::2] | (seg[1::2] << 4)                     # 16 bytes
        words = by.reshape(4, 4)
        regs[l, :4] = words[:, 0] | (words[:, 1] << 8) | (words[:, 2] << 16) | (words[:, 3] << 24)
    return regs.view(np.int32)


def _close(got, expect, a, a_sc, b, b_sc):
    """float32 accumulation of exact products: within K * 2^-24 of sum |a b|
    (a wrong lane mapping misses by O(1) relative)."""
    aa = np.abs(oracle.e2m1_decode(a)) * np.repeat(oracle.e8m0_decode(a_sc), 32, axis=1)
    bb = np.abs(oracle.e2m1_decode(b)) * np.repeat(oracle.e8m0_decode(b_sc), 32, axis=1)
    bound = aa @ bb.T
    assert np.all(np.abs(got - expect) <= a.shape[1] * 2.0 ** -24 * bound)


def _model(a_codes, a_sc, b_codes, b_sc):
    a = oracle.e2m1_decode(a_codes) * np.repeat(oracle.e8m0_decode(a_sc), 32, axis=1)
    b = oracle.e2m1_decode(b_codes) * np.repeat(oracle.e8m0_decode(b_sc), 32, axis=1)
    return a @ b.T


@pytest.mark.parametrize("opsel2", [0, 1])
def test_mfma_scale_32x32x64_layout(opsel2):
    need_gpu()
    lib = probe_lib()
    rng = np.random.default_rng(100 + opsel2)
    a = rng.integers(0, 16, size=(32, 64))
    b = rng.integers(0, 16, size=(32, 64))
    a_sc = rng.integers(120, 135, size=(32, 2))
    b_sc = rng.integers(120, 135, size=(32, 2))
    # scale words: the used byte is 0 (op_sel 0) or 2 (op_sel 2); other bytes are junk
    sa = rng.integers(0, 2**31, size=64).astype(np.int64)
    sb = rng.integers(0, 2**31, size=64).astype(np.int64)
    sh = 16 if opsel2 else 0
    for l in range(64):
        sa[l] = (sa[l] & ~(0xFF << sh)) | (int(a_sc[l % 32, l // 32]) << sh)
        sb[l] = (sb[l] & ~(0xFF << sh)) | (int(b_sc[l % 32, l // 32]) << sh)
    ar = torch.from_numpy(_lane_regs(a, 32, 2)).cuda()
    br = torch.from_numpy(_lane_regs(b, 32, 2)).cuda()
    sat = torch.from_numpy(sa.astype(np.uint32).view(np.int32)).cuda()
    sbt = torch.from_numpy(sb.astype(np.uint32).view(np.int32)).cuda()
    out = torch.zeros(64 * 16, dtype=torch.float32, device="cuda")
    banner(f"mfma 32x32x64 opsel2={opsel2}")
    assert lib.probe_mfma_scale_32x32x64(ar.data_ptr(), br.data_ptr(), sat.data_ptr(),
                                         sbt.data_ptr(), out.data_ptr(), opsel2) == 0
    torch.cuda.synchronize()
    raw = out.cpu().numpy().reshape(64, 16)
    expect = _model(a, a_sc, b, b_sc)
    got = np.zeros((32, 32))
    for l in range(64):
        for r in range(16):
            got[8 * (r // 4) + 4 * (l // 32) + (r % 4), l % 32] = raw[l, r]
    save_npz(f"probe_mfma32_{opsel2}.npz", a=a, b=b, a_sc=a_sc, b_sc=b_sc, raw=raw, expect=expect)
    _close(got, expect, a, a_sc, b, b_sc)


_FMT = {"e4m3": 0, "e5m2": 1, "e2m3": 2, "e3m2": 3, "e2m1": 4}


def _finite_codes(rng, elem, shape):
    """Random finite codes of an element type (no NaN/Inf encodings)."""
    if elem == "e2m1":
        return rng.integers(0, 16, size=shape)
    e, m, top = oracle.elements.ELEMS[elem]
    mag = rng.integers(0, top + 1, size=shape)
    return mag | (rng.integers(0, 2, size=shape) << (e + m))


def _pack_row_bytes(codes, elem):
    if elem == "e2m1":
        return oracle.pack_nibbles(codes)
    return oracle.elements.pack(codes, elem)


def _fmt_lane_regs(codes, elem):
    """Per-lane 8 x int32 registers of row l % 32, g = l // 32, taken from the
    operand's storage bytes: FP4 and FP6, the bytes of K-block g (elements
    [32g, 32g+32): 16 or 24 bytes); FP8, two 16-element halves, elements
    [16g, 16g+16) then [32+16g, 48+16g) (2 x 16 bytes); the rest zero."""
    packed = _pack_row_bytes(codes, elem)            # [32, 64 * bits / 8]
    bits = 4 if elem == "e2m1" else oracle.elements.elem_bits(elem)
    regs = np.zeros((64, 32), dtype=np.uint8)
    for l in range(64):
        r, g = l % 32, l // 32
        if bits == 8:
            regs[l, :16] = packed[r, 16 * g:16 * g + 16]
            regs[l, 16:32] = packed[r, 32 + 16 * g:48 + 16 * g]
        else:
            bpb = 4 * bits                           # bytes per 32 elements
            regs[l, :bpb] = packed[r, g * bpb:(g + 1) * bpb]
    return regs.view(np.int32).reshape(64, 8)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e2m3", "e2m3"), ("e3m2", "e3m2"),
                                   ("e4m3", "e2m1"), ("e2m1", "e3m2"), ("e5m2", "e2m3")])
def test_mfma_scale_32x32x64_element_formats(fa, fb):
    """The instruction's FP8 and FP6 operand layout: with the library's storage
    (FP8: byte i = element i; FP6: element i at bits 6i of the row,
    little-endian; FP4: two per byte, low nibble first) a lane of K-half g
    takes, for FP8, the 16-element halves [16g, 16g+16) and [32+16g, 48+16g),
    for FP6 and FP4 the whole block [32g, 32g+32); its scale byte is that of
    K-block g either way.  The result equals the oracle's reference within the
    instruction's internal precision (mx_group_bound), mixed formats included."""
    need_gpu()
    lib = probe_lib()
    rng = np.random.default_rng(_FMT[fa] * 10 + _FMT[fb])
    a = _finite_codes(rng, fa, (32, 64))
    b = _finite_codes(rng, fb, (32, 64))
    a_sc = rng.integers(120, 135, size=(32, 2)).astype(np.uint8)
    b_sc = rng.integers(120, 135, size=(32, 2)).astype(np.uint8)
    sa = np.array([a_sc[l % 32, l // 32] for l in range(64)], dtype=np.int32)
    sb = np.array([b_sc[l % 32, l // 32] for l in range(64)], dtype=np.int32)
    ar = torch.from_numpy(_fmt_lane_regs(a, fa)).cuda()
    br = torch.from_numpy(_fmt_lane_regs(b, fb)).cuda()
    out = torch.zeros(64 * 16, dtype=torch.float32, device="cuda")
    banner(f"mfma 32x32x64 formats {fa} x {fb}")
    assert lib.probe_mfma_scale_32x32x64_fmt(ar.data_ptr(), br.data_ptr(), torch.from_numpy(sa).cuda().data_ptr(),
                                             torch.from_numpy(sb).cuda().data_ptr(), out.data_ptr(),
                                             _FMT[fa], _FMT[fb]) == 0
    torch.cuda.synchronize()
    raw = out.cpu().numpy().reshape(64, 16)
    got = np.zeros((32, 32))
    for l in range(64):
        for r in range(16):
            got[8 * (r // 4) + 4 * (l // 32) + (r % 4), l % 32] = raw[l, r]
    ref, bound = oracle.gemm_ref(_pack_row_bytes(a, fa), a_sc, _pack_row_bytes(b, fb), b_sc,
                                 a_elem=fa, b_elem=fb)
    save_npz(f"probe_mfma_fmt_{fa}_{fb}.npz", raw=raw, ref=ref)
    av = oracle.gemm.dequant_f64(_pack_row_bytes(a, fa), a_sc, fa)
    bv = oracle.gemm.dequant_f64(_pack_row_bytes(b, fb), b_sc, fb)
    tol = 64 * 2.0 ** -24 * bound + mx_group_bound(av, bv)
    assert np.all(np.abs(got - ref) <= tol), float(np.max(np.abs(got - ref) / tol))


def test_mfma_scale_16x16x128_layout():
    need_gpu()
    lib = probe_lib()
    rng = np.random.default_rng(7)
    a = rng.integers(0, 16, size=(16, 128))
    b = rng.integers(0, 16, size=(16, 128))
    a_sc = rng.integers(120, 135, size=(16, 4))
    b_sc = rng.integers(120, 135, size=(16, 4))
    sa = np.array([a_sc[l % 16, l // 16] for l in range(64)], dtype=np.int32)
    sb = np.array([b_sc[l % 16, l // 16] for l in range(64)], dtype=np.int32)
    ar = torch.from_numpy(_lane_regs(a, 16, 4)).cuda()
    br = torch.from_numpy(_lane_regs(b, 16, 4)).cuda()
    out = torch.zeros(64 * 4, dtype=torch.float32, device="cuda")
    banner("mfma 16x16x128")
    assert lib.probe_mfma_scale_16x16x128(ar.data_ptr(), br.data_ptr(),
                                          torch.from_numpy(sa).cuda().data_ptr(),
                                          torch.from_numpy(sb).cuda().data_ptr(),
                                          out.data_ptr()) == 0
    torch.cuda.synchronize()
    raw = out.cpu().numpy().reshape(64, 4)
    expect = _model(a, a_sc, b, b_sc)
    got = np.zeros((16, 16))
    for l in range(64):
        for r in range(4):
            got[4 * (l // 16) + r, l % 16] = raw[l, r]
    save_npz("probe_mfma16.npz", a=a, b=b, a_sc=a_sc, b_sc=b_sc, raw=raw, expect=expect)
    _close(got, expect, a, a_sc, b, b_sc)


def _sweep(lib, lo, hi, cap=64):
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    first = torch.zeros(2 * cap, dtype=torch.int32, device="cuda")
    assert lib.probe_cvt_fp4_sweep(lo, hi, cnt.data_ptr(), first.data_ptr(), cap) == 0
    torch.cuda.synchronize()
    n = int(cnt[0].item())
    f = first.cpu().numpy().view(np.uint32).reshape(cap, 2)[:min(n, cap)]
    return n, f


def test_hw_fp4_cvt_matches_software_rne_everywhere():
    """The hardware conversion with scale 1.0 equals the software RNE
    (saturation, ties to even, signed zero, subnormals) for every non-NaN
    float32 x and -x."""
    need_gpu()
    lib = probe_lib()
    banner("cvt sweep [0, 8)")
    n_in, f_in = _sweep(lib, 0, 0x41000000)
    banner("cvt sweep [8, inf]")
    n_out, f_out = _sweep(lib, 0x41000000, 0x7F800001)
    save_npz("probe_cvt.npz", n_in=n_in, f_in=f_in, n_out=n_out, f_out=f_out)
    print(f"hw-vs-sw fp4 cvt mismatches: |x|<8: {n_in}, |x|>=8: {n_out}")
    for u, code in list(f_in[:8]) + list(f_out[:8]):
        print(f"  x=0x{u:08x} ({np.uint32(u).view(np.float32)!r}) hw=0x{code & 0xFF:02x} sw=0x{code >> 8:02x}")
    assert n_in == 0 and n_out == 0


@pytest.mark.parametrize("k", [-127, -126, -100, -60, -3, -1, 0, 1, 2, 17, 90, 124, 125, 126])
def test_hw_fp4_cvt_scale_operand_divides(k):
    """With a power-of-two scale 2^k the instruction returns exactly
    RNE_fp4(RNE_fp32(x * 2^-k)) for every non-NaN x: the quantizer hands it the
    block scale instead of multiplying first (scale bytes >= 1; 2^126 is the
    largest scale the round-up rule gives).  The lowest scale byte, whose
    2^-127 is a float32 subnormal, is asserted as well, although no kernel
    passes it: they multiply by 2^127 and convert at scale 1 instead."""
    need_gpu()
    lib = probe_lib()
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    banner(f"cvt scaled sweep k={k}")
    assert lib.probe_cvt_fp4_scaled_sweep(0, 0x7F800001, k, cnt.data_ptr()) == 0
    torch.cuda.synchronize()
    c = cnt.cpu().numpy()
    print(f"cvt scale 2^{k}: mismatches vs divide={c[0]} vs multiply={c[1]}")
    save_npz(f"probe_cvt_scale_{k}.npz", counts=c)
    assert c[0] == 0


def test_hw_fp4_sr_matches_software_sr_everywhere():
    """pack8_sr (the hardware SR conversion on sign(v) ceil(|v| 2^23) with
    scale 2^23, one draw per element) equals e2m1_sr for every float32 with
    |x| < 8 (x and -x, all four byte positions), at draws T-1, T, T+1 around
    the threshold T = floor(f 2^16) and at hashed draws."""
    need_gpu()
    lib = probe_lib()
    cap = 32
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    first = torch.zeros(3 * cap, dtype=torch.int32, device="cuda")
    banner("cvt sr sweep [0, 8)")
    assert lib.probe_cvt_fp4_sr_sweep(0, 0x41000000, cnt.data_ptr(), first.data_ptr(), cap) == 0
    torch.cuda.synchronize()
    n = int(cnt[0].item())
    f = first.cpu().numpy().view(np.uint32).reshape(cap, 3)[:min(n, cap)]
    save_npz("probe_cvt_sr.npz", n=n, first=f)
    print(f"hw-vs-sw fp4 SR mismatches: {n}")
    for u, hw, sw in f[:8]:
        print(f"  x=0x{u:08x} ({np.uint32(u).view(np.float32)!r}) hw=0x{hw:08x} sw=0x{sw:08x}")
    assert n == 0


def _fp_sweep(fn, lo, hi, elem, k, width):
    cap = 16
    cnt = torch.zeros(3, dtype=torch.int64, device="cuda")
    first = torch.zeros(width * cap, dtype=torch.int32, device="cuda")
    assert fn(lo, hi, elem, k, cnt.data_ptr(), first.data_ptr(), cap) == 0
    torch.cuda.synchronize()
    c = cnt.cpu().numpy()
    f = first.cpu().numpy().view(np.uint32).reshape(cap, width)[:min(int(c[2]), cap)]
    return c, f


@pytest.mark.parametrize("elem", [1, 2])
@pytest.mark.parametrize("k", [-126, -20, 0, 3, 100, 125])
def test_hw_fp8_pack_matches_software_rne(elem, k):
    """mx::pack4_fp8 (V_CVT_SCALEF32_PK_FP8/BF8_F32 with scale 2^k on inputs
    clamped to +-(largest normal * 2^k)) equals the software RNE codes of
    x / 2^k (E4M3 / E5M2, saturating) in all four bytes, for every finite
    float32 x >= 0 (and -x; a block holding Inf or NaN gets the NaN scale and
    no conversion).  Mismatches are counted apart for
    |x| / 2^k >= 2^(emax+1), which no block holds after division by its scale."""
    need_gpu()
    lib = probe_lib()
    banner(f"fp8 cvt sweep elem={elem} k={k}")
    c, f = _fp_sweep(lib.probe_cvt_fp8_sweep, 0, 0x7F800000, elem, k, 3)
    save_npz(f"probe_cvt_fp8_{elem}_{k}.npz", counts=c, first=f)
    print(f"fp8 elem {elem} scale 2^{k}: mismatches in range {c[0]}, above {c[1]}")
    for u, hw, sw in f[:8]:
        print(f"  x=0x{u:08x} ({np.uint32(u).view(np.float32)!r}) hw=0x{hw:08x} sw=0x{sw:08x}")
    assert c[0] == 0 and c[1] == 0


@pytest.mark.parametrize("elem", [3, 4])
@pytest.mark.parametrize("k", [-126, 0, 7, 125])
def test_hw_fp6_pack_matches_software_rne_and_packing(elem, k):
    """mx::pack32_fp6 (V_CVT_SCALEF32_2XPK16_FP6/BF6_F32, 32 values, scale 2^k,
    clamped inputs) equals the software RNE codes of x / 2^k packed 6 bits per
    element, element e at bit 6e (E2M3 / E3M2), over every finite float32
    pattern in groups of 32 with alternating signs."""
    need_gpu()
    lib = probe_lib()
    banner(f"fp6 cvt sweep elem={elem} k={k}")
    c, f = _fp_sweep(lib.probe_cvt_fp6_sweep, 0, 0x7F800000, elem, k, 13)
    save_npz(f"probe_cvt_fp6_{elem}_{k}.npz", counts=c, first=f)
    print(f"fp6 elem {elem} scale 2^{k}: mismatching groups in range {c[0]}, above {c[1]}")
    for row in f[:4]:
        print(f"  x=0x{row[0]:08x} hw={[hex(v) for v in row[1:7]]} sw={[hex(v) for v in row[7:13]]}")
    assert c[0] == 0 and c[1] == 0
