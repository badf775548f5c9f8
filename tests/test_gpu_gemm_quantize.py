"""GPU parity of mx_gemm_quantize, the GEMM whose epilogue quantizes the
product along N into MXFP4 (1-D blocks, RNE) instead of storing it.

Three checks per case:
* bit-exact against the unfused composition on the same device: mx_gemm with
  float32 output (the same MFMA accumulation, so the same float32 values)
  followed by mx_quantize of that output along its last dim;
* against the oracle from the operands alone: every scale byte and code must
  be the oracle's quantization of some product within the GEMM error bound of
  its float64 reference (exactly the oracle's answer wherever no scale or
  rounding boundary lies inside the bound; no GPU value enters the oracle);
* the float32 product itself against that reference within the bound.
Padding bytes of the output rows are filled with a marker and must survive.
"""
import zlib

import numpy as np
import pytest
import torch

import mxfp4_microscaling_quantization_mx_amd as mx
import oracle
import workloads
from gpu_util import banner, check_gemm, check_quantized_product, codes_equal, host, mx_group_bound, need_gpu
from test_gpu_elements import _operand
from test_gpu_gemm import _rand_mx, _upload

pytestmark = pytest.mark.gpu


def _full_rows(t):
    return t.as_strided((t.shape[0], t.stride(0)), (t.stride(0), 1))


def _marked_out(M, N, fill=0x5A):
    q = mx.empty_mx(M, N)
    _full_rows(q.codes).fill_(fill)
    _full_rows(q.scales).fill_(fill)
    return q


def _check_fused(a, b, M, N, scale_mode, ref_inputs):
    fused = _marked_out(M, N)
    mx.gemm_quantize(a, b, scale_mode=scale_mode, out=fused)
    y = mx.gemm(a, b, torch.float32)
    unfused = mx.quantize(y, scale_mode=scale_mode)
    fc, fs = host(fused.codes), host(fused.scales)
    codes_equal(fc, host(unfused.codes), "codes vs gemm + quantize")
    codes_equal(fs, host(unfused.scales), "scales vs gemm + quantize")
    yn = host(y)
    assert np.all(host(_full_rows(fused.codes))[:, N // 2:] == 0x5A), "code row padding written"
    assert np.all(host(_full_rows(fused.scales))[:, N // 32:] == 0x5A), "scale row padding written"
    ref, bound = oracle.gemm_ref(*ref_inputs)
    check_gemm(yn, ref, bound, what="product")
    fin = np.isfinite(ref).all(axis=1)            # NaN rows are checked by their own test
    K = ref_inputs[0].shape[1] * 2
    check_quantized_product(fc[fin], fs[fin], ref[fin], bound[fin], K, scale_mode)
    return fc, fs


@pytest.mark.parametrize("M,N,K,a_block,b_block", [
    (256, 256, 128, "1d", "1d"),
    (300, 544, 224, "1d", "1d"),       # ragged M, N not a multiple of 256, K tail inside a stage
    (520, 800, 2880, "1d", "2d"),      # several tiles, 2-D weight scales, the fprop K
    (512, 288, 352, "2d", "1d"),
])
@pytest.mark.parametrize("scale_mode", ["floor", "round_up", "prescale_3_4"])
def test_gemm_quantize_matches_unfused_and_oracle(M, N, K, a_block, b_block, scale_mode):
    need_gpu()
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    ac, as_ = _rand_mx(rng, M, K, a_block)
    bc, bs = _rand_mx(rng, N, K, b_block)
    banner(f"gemm_quantize M={M} N={N} K={K} {a_block}/{b_block} {scale_mode}")
    _check_fused(_upload(ac, as_, a_block), _upload(bc, bs, b_block), M, N, scale_mode,
                 (ac, as_, bc, bs, a_block, b_block))


def test_gemm_quantize_nan_and_zero_rows():
    """A NaN scale poisons its rows (scale byte 0xFF, zero codes, as the
    quantizer does for a block with NaN); all-zero rows get scale byte 0."""
    need_gpu()
    rng = np.random.default_rng(11)
    ac, as_ = _rand_mx(rng, 256, 256)
    bc, bs = _rand_mx(rng, 256, 256)
    as_[17, 3] = 0xFF
    ac[40] = 0
    banner("gemm_quantize nan / zero rows")
    fc, fs = _check_fused(_upload(ac, as_), _upload(bc, bs), 256, 256, "floor",
                          (ac, as_, bc, bs, "1d", "1d"))
    assert np.all(fs[17] == 0xFF) and np.all(fc[17] == 0)
    assert np.all(fs[40] == 0) and np.all(fc[40] == 0)


def test_gemm_quantize_scale_byte_zero_blocks():
    """Products whose 32-column block maximum lies below 2^-124 take the
    lowest scale byte (exponent -127; "MXFP4", AI Wiki, §Format specification:
    E8M0 range) and still carry non-zero codes: each value is divided by
    2^-127 exactly before rounding.  A scales of 17 .. 25 with B scales of 100
    put the block maxima around 2^-126 .. 2^-121, so both byte 0 and the bytes
    above it occur, with float32 subnormal products among them."""
    need_gpu()
    rng = np.random.default_rng(12)
    M, N, K = 256, 288, 256
    ac, as_ = _rand_mx(rng, M, K)
    bc, bs = _rand_mx(rng, N, K)
    as_[:] = rng.integers(17, 26, as_.shape).astype(np.uint8)
    bs[:] = 100
    banner("gemm_quantize scale byte 0 blocks")
    fc, fs = _check_fused(_upload(ac, as_), _upload(bc, bs), M, N, "floor", (ac, as_, bc, bs, "1d", "1d"))
    zero = fs == 0
    codes = oracle.unpack_nibbles(fc).reshape(M, N // 32, 32)
    assert zero.sum() > 50 and (~zero).sum() > 50
    assert np.count_nonzero(codes[zero] & 7) > 1000, "byte-0 blocks should hold non-zero codes"


def test_gemm_quantize_zero_k():
    """K = 0: the product is zero, so every block gets scale byte 0 and zero
    codes (what mx_quantize gives for zeros)."""
    need_gpu()
    banner("gemm_quantize K=0")
    out = _marked_out(256, 288)
    mx.gemm_quantize(mx.empty_mx(256, 0), mx.empty_mx(288, 0), out=out)
    assert np.all(host(out.codes) == 0) and np.all(host(out.scales) == 0)


def test_gemm_quantize_fprop_full_size():
    """The fprop workload (X 16384x2880 with the transform, W 2880x5760 in 2-D
    tiles, both RNE) with its output quantized in the epilogue: the whole
    16384 x 5760 result equals mx_gemm (float32) + mx_quantize bit for bit, and
    48 sampled rows x two 32-column blocks are the oracle's quantization of the
    reference product within its bound."""
    need_gpu()
    x, w = workloads.fprop()
    mask = workloads.rht_mask(workloads.CFG_FPROP)
    banner("gemm_quantize fprop full size")
    qx = mx.quantize(x.cuda(), rht_mask=mask)
    qw = mx.quantize(w.cuda(), axis="dim0", block="2d", rht_mask=mask)
    fused = mx.gemm_quantize(qx, qw)
    y = mx.gemm(qx, qw, torch.float32)
    unfused = mx.quantize(y)
    assert torch.equal(fused.codes, unfused.codes) and torch.equal(fused.scales, unfused.scales)
    rng = np.random.default_rng(4)
    rows = np.sort(rng.choice(16384, 48, replace=False))
    blocks = np.sort(rng.choice(5760 // 32, 2, replace=False))
    cols = (blocks[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    xn, wn = x.float().numpy(), w.float().numpy()
    oxc, oxs = oracle.quantize(xn[rows], rht_mask=mask)
    owc, ows = oracle.quantize(wn[:, cols], axis="dim0", block="2d", rht_mask=mask)
    ref, bound = oracle.gemm_ref(oxc, oxs, owc, ows, "1d", "2d")
    bytes_ = (blocks[:, None] * 16 + np.arange(16)[None, :]).reshape(-1)
    check_quantized_product(host(fused.codes)[np.ix_(rows, bytes_)], host(fused.scales)[np.ix_(rows, blocks)],
                            ref, bound, 2880, what="fprop sampled rows")


# ---------------------------------------------------------------- grouped
def _grouped_operands(rng, offsets, N, K, M_cap):
    E = len(offsets) - 1
    ac, as_ = _rand_mx(rng, M_cap, K)
    bcs, bss = zip(*[_rand_mx(rng, N, K, "2d") for _ in range(E)])
    bc, bs = np.stack(bcs), np.stack(bss)
    a = _upload(ac, as_)
    ld = (bs.shape[2] + 15) // 16 * 16
    buf = torch.full((E, bs.shape[1], ld), 0xFF, dtype=torch.uint8, device="cuda")
    buf[:, :, :bs.shape[2]] = torch.from_numpy(bs).cuda()
    b = mx.MXTensor(torch.from_numpy(bc).cuda(), buf[:, :, :bs.shape[2]], N, K, "2d")
    return a, b, (ac, as_, bc, bs)


@pytest.mark.parametrize("offsets,M_cap", [([0, 5, 5, 300, 333], 400), ([0, 600], 600),
                                           ([0, 0, 0, 257, 257, 800], 800), ([0, 1, 2, 3, 4, 260, 261, 700], 720)])
@pytest.mark.parametrize("N,K", [(288, 2880), (544, 416)])
@pytest.mark.parametrize("scale_mode", ["floor", "round_up"])
def test_grouped_gemm_quantize_matches_unfused(offsets, M_cap, N, K, scale_mode):
    """Grouped product quantized in the epilogue (empty experts, 1-row experts,
    tiles straddling expert boundaries, ragged N and K): rows [0, off[E])
    equal mx_grouped_gemm (float32) + mx_quantize bit for bit and the oracle's
    quantization of the reference product within its bound; rows past off[E]
    keep the marker."""
    need_gpu()
    rng = np.random.default_rng(len(offsets) * 17 + offsets[-1] + N + K)
    a, b, (ac, as_, bc, bs) = _grouped_operands(rng, offsets, N, K, M_cap)
    off = torch.from_numpy(np.asarray(offsets, dtype=np.int32)).cuda()
    banner(f"grouped_gemm_quantize offsets={offsets} N={N} K={K} {scale_mode}")
    fused = _marked_out(M_cap, N)
    mx.grouped_gemm_quantize(a, off, b, scale_mode=scale_mode, out=fused)
    m = offsets[-1]
    y = mx.grouped_gemm(a, off, b, torch.float32)
    yh = host(y)[:m]
    unfused = mx.quantize(y[:m].contiguous(), scale_mode=scale_mode)
    fc, fs = host(fused.codes), host(fused.scales)
    codes_equal(fc[:m], host(unfused.codes), "codes vs grouped_gemm + quantize")
    codes_equal(fs[:m], host(unfused.scales), "scales vs grouped_gemm + quantize")
    assert np.all(fc[m:] == 0x5A) and np.all(fs[m:] == 0x5A), "rows past the last offset written"
    ref, bound = oracle.grouped_gemm_ref(ac[:m], as_[:m], offsets, bc, bs)
    check_gemm(yh, ref, bound, what="grouped product")
    check_quantized_product(fc[:m], fs[:m], ref, bound, K, scale_mode, what="grouped")


def test_grouped_gemm_quantize_moe_full_size():
    """The MoE workload's grouped product (65536 routed rows x 5760, 32 experts,
    Zipf 1.1 top-4) quantized in the epilogue equals mx_grouped_gemm (float32)
    + mx_quantize over the whole output, and sampled rows of two experts (two
    32-column blocks each) are the oracle's quantization of the reference
    product within its bound."""
    need_gpu()
    tok, offsets = workloads.moe_routing()
    E, K, N = 32, 2880, 5760
    banner("grouped_gemm_quantize moe full size")
    xc = workloads.to_bf16(workloads.moe_tokens())
    x = xc.cuda()
    qa = mx.quantize_gather(x, torch.from_numpy(tok.astype(np.int32)).cuda())
    qb = mx.empty_mx(N, K, "2d", experts=E)
    for e in range(E):
        we = workloads.to_bf16(workloads.moe_expert_weight(e)).cuda()
        mx.quantize(we, axis="dim0", block="2d", out=mx.expert(qb, e))
    off = torch.from_numpy(np.asarray(offsets, dtype=np.int32)).cuda()
    fused = mx.grouped_gemm_quantize(qa, off, qb)
    y = mx.grouped_gemm(qa, off, qb, torch.float32)
    unfused = mx.quantize(y)
    assert torch.equal(fused.codes, unfused.codes) and torch.equal(fused.scales, unfused.scales)
    rng = np.random.default_rng(8)
    xn = xc.float().numpy()
    fc, fs = host(fused.codes), host(fused.scales)
    for e in [int(np.argmax(np.diff(offsets))), 5]:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        rows = np.sort(rng.choice(np.arange(lo, hi), min(16, hi - lo), replace=False))
        blocks = np.sort(rng.choice(N // 32, 2, replace=False))
        cols = (blocks[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
        wn = workloads.to_bf16(workloads.moe_expert_weight(e)).float().numpy()
        oac, oas = oracle.quantize(xn[tok[rows]])
        owc, ows = oracle.quantize(wn[:, cols], axis="dim0", block="2d")
        ref, bound = oracle.gemm_ref(oac, oas, owc, ows, "1d", "2d")
        bytes_ = (blocks[:, None] * 16 + np.arange(16)[None, :]).reshape(-1)
        check_quantized_product(fc[np.ix_(rows, bytes_)], fs[np.ix_(rows, blocks)], ref, bound, K,
                                what=f"moe expert {e}")


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e3m2"), ("e2m3", "e2m3"), ("e3m2", "e4m3")])
@pytest.mark.parametrize("M,N,K,b_block", [(256, 256, 256, "1d"), (300, 544, 224, "2d"), (520, 800, 2880, "2d")])
def test_gemm_quantize_mxfp8_mxfp6(fa, fb, M, N, K, b_block):
    """MXFP8 / MXFP6 operands ("MXFP4", AI Wiki, §Place in the MX family) with
    the product quantized to MXFP4 in the epilogue of their direct-to-LDS
    kernel: bit-exact against mx_gemm (float32) + mx_quantize (the same MFMAs
    with the operands exchanged), padding untouched, and against the oracle
    within the GEMM bound plus the instruction's alignment allowance."""
    need_gpu()
    rng = np.random.default_rng(zlib.crc32(f"q{fa}{fb}{M}{N}{K}".encode()))
    qa, ac, as_ = _operand(rng, M, K, fa)
    qb, bc, bs = _operand(rng, N, K, fb, b_block)
    banner(f"gemm_quantize {fa} x {fb} M={M} N={N} K={K} {b_block}")
    fused = _marked_out(M, N)
    mx.gemm_quantize(qa, qb, out=fused)
    y = mx.gemm(qa, qb, torch.float32)
    unfused = mx.quantize(y)
    fc, fs = host(fused.codes), host(fused.scales)
    codes_equal(fc, host(unfused.codes), "codes vs gemm + quantize")
    codes_equal(fs, host(unfused.scales), "scales vs gemm + quantize")
    assert np.all(host(_full_rows(fused.codes))[:, N // 2:] == 0x5A), "code row padding written"
    assert np.all(host(_full_rows(fused.scales))[:, N // 32:] == 0x5A), "scale row padding written"
    ref, bound = oracle.gemm_ref(ac, as_, bc, bs, "1d", b_block, a_elem=fa, b_elem=fb)
    gb = mx_group_bound(oracle.gemm.dequant_f64(ac, as_, fa), oracle.gemm.dequant_f64(bc, bs, fb, b_block))
    check_quantized_product(fc, fs, ref, bound, K, extra=gb)


def test_gemm_quantize_mixed_fp4_rejected():
    """One MXFP4 and one MXFP8 operand: MX_ERR_UNSUPPORTED, nothing written."""
    need_gpu()
    rng = np.random.default_rng(5)
    qa, _, _ = _operand(rng, 256, 256, "e2m1")
    qb, _, _ = _operand(rng, 256, 256, "e4m3")
    out = _marked_out(256, 256)
    with pytest.raises(mx.MXError):
        mx.gemm_quantize(qa, qb, out=out)
    assert np.all(host(_full_rows(out.codes)) == 0x5A)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e2m3", "e5m2")])
@pytest.mark.parametrize("N", [256, 544])
def test_grouped_gemm_quantize_mxfp8_mxfp6(fa, fb, N):
    """Grouped MXFP8 / MXFP6 product quantized to MXFP4 in the epilogue
    (empty experts, a one-row expert, experts straddling row tiles): routed
    rows equal mx_grouped_gemm (float32) + mx_quantize bit for bit and the
    oracle's quantization of the reference within its bound plus the
    alignment allowance; rows past the last offset keep the marker."""
    from test_gpu_elements import _finite_codes, _pack
    from gpu_util import to_dev
    need_gpu()
    rng = np.random.default_rng(zlib.crc32(f"gq{fa}{fb}{N}".encode()))
    offsets = np.array([0, 0, 1, 300, 300, 557, 700], dtype=np.int32)
    E, K, M = len(offsets) - 1, 224, 720
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
    off = torch.from_numpy(offsets).cuda()
    banner(f"grouped_gemm_quantize {fa} x {fb} N={N}")
    fused = _marked_out(M, N)
    mx.grouped_gemm_quantize(qa, off, qb, out=fused)
    m = int(offsets[-1])
    y = mx.grouped_gemm(qa, off, qb, torch.float32)
    unfused = mx.quantize(y[:m].contiguous())
    fc, fs = host(fused.codes), host(fused.scales)
    codes_equal(fc[:m], host(unfused.codes), "codes vs grouped_gemm + quantize")
    codes_equal(fs[:m], host(unfused.scales), "scales vs grouped_gemm + quantize")
    assert np.all(fc[m:] == 0x5A) and np.all(fs[m:] == 0x5A), "rows past the last offset written"
    ref, bound = oracle.grouped_gemm_ref(ac, as_, offsets, bc, bs, "1d", "2d", rows=np.arange(m),
                                         a_elem=fa, b_elem=fb)
    av = oracle.gemm.dequant_f64(ac[:m], as_[:m], fa)
    gb = np.zeros_like(bound)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            gb[lo:hi] = mx_group_bound(av[lo:hi], oracle.gemm.dequant_f64(bc[e], bs[e], fb, "2d"))
    check_quantized_product(fc[:m], fs[:m], ref, bound, K, extra=gb, what="grouped mxfp8/6")
