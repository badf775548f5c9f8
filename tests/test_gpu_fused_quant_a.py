"""GPU parity of mx_gemm_fused_quant_a: the A operand handed over in bf16 and
quantized to MXFP4 inside the GEMM's operand load.

Its blocks are quantized by the quantizer's own rule ("MXFP4", AI Wiki,
§Conversion rules and §Clipping in the reference algorithm), so on shapes that
mx_gemm does not split along K the result must equal, bit for bit, mx_gemm of
mx_quantize(A) (both accumulate one 64-deep step at a time in K order).  Every
case is also held to the GEMM rule of the other tests against the oracle:
|C - ref| <= 1e-5 * sum_k |a_k b_k|, ref the float64 product of the oracle's
quantization of the same bf16 rows.
"""
import numpy as np
import pytest
import torch

import mxfp4_microscaling_quantization_mx_amd as mx
import oracle
from gpu_util import banner, check_gemm, host, need_gpu

pytestmark = pytest.mark.gpu


def _inputs(seed, M, N, K, b_block="1d"):
    rng = np.random.default_rng(seed)
    a = (rng.standard_t(3, (M, K)) * np.exp(rng.uniform(-3, 3, (M, 1)))).astype(np.float32)
    at = torch.from_numpy(a).to(torch.bfloat16)
    w = rng.standard_normal((N, K)).astype(np.float32)
    wt = torch.from_numpy(w).to(torch.bfloat16)
    return at, wt


def _splits(M, N, K):
    return mx.load_library().mx_gemm_workspace_size(M, N, K) > 0


@pytest.mark.parametrize("M,N,K", [(1000, 700, 96), (2341, 4112, 1056), (300, 520, 4128)])
@pytest.mark.parametrize("rht", [False, True])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fused_quant_a_matches_unfused_and_oracle(M, N, K, rht, out_dtype):
    """Ragged M, N and K tails (K = 1056 ends one block into a 128-deep
    stage); with and without the transform; both output types."""
    need_gpu()
    at, wt = _inputs(M + 3 * N + 7 * K + int(rht), M, N, K)
    mask = 0x6B8B4567 if rht else None
    banner(f"fused quant A M={M} N={N} K={K} rht={rht} {out_dtype}")
    ad = at.cuda()
    qb = mx.quantize(wt.cuda(), rht_mask=mask)
    c = mx.gemm_fused_quant_a(ad, qb, out_dtype, rht_mask=mask)
    unfused = mx.gemm(mx.quantize(ad, rht_mask=mask), qb, out_dtype)
    if not _splits(M, N, K):
        assert torch.equal(c.view(torch.int16) if out_dtype == torch.bfloat16 else c.view(torch.int32),
                           unfused.view(torch.int16) if out_dtype == torch.bfloat16 else unfused.view(torch.int32)), \
            "differs from mx_quantize + mx_gemm"
    rows = np.arange(M) if M * N <= 1_000_000 else np.sort(np.random.default_rng(1).choice(M, 96, replace=False))
    an, wn = at.float().numpy(), wt.float().numpy()
    ac, as_ = oracle.quantize(an[rows], rht_mask=mask)
    bc, bs = oracle.quantize(wn, rht_mask=mask)
    ref, bound = oracle.gemm_ref(ac, as_, bc, bs)
    check_gemm(host(c.float())[rows], ref, bound, bf16=(out_dtype == torch.bfloat16), what="fused quant A")


@pytest.mark.parametrize("scale_mode", ["round_up", "prescale_3_4"])
def test_fused_quant_a_scale_modes(scale_mode):
    need_gpu()
    M, N, K = 1000, 700, 96
    at, wt = _inputs(11, M, N, K)
    banner(f"fused quant A scale mode {scale_mode}")
    ad = at.cuda()
    qb = mx.quantize(wt.cuda())
    c = mx.gemm_fused_quant_a(ad, qb, torch.float32, scale_mode=scale_mode)
    unfused = mx.gemm(mx.quantize(ad, scale_mode=scale_mode), qb, torch.float32)
    assert torch.equal(c.view(torch.int32), unfused.view(torch.int32))
    ac, as_ = oracle.quantize(at.float().numpy(), scale_mode=scale_mode)
    bc, bs = oracle.quantize(wt.float().numpy())
    ref, bound = oracle.gemm_ref(ac, as_, bc, bs)
    check_gemm(host(c), ref, bound, what=f"fused quant A {scale_mode}")


def test_fused_quant_a_2d_weight_and_guard_rows():
    """B with 32x32 blocks (the weight layout), C inside a larger buffer filled
    with a marker: nothing outside C is written."""
    need_gpu()
    M, N, K = 1000, 704, 640
    at, wt = _inputs(12, M, N, K)
    banner("fused quant A 2-D B, guarded C")
    ad = at.cuda()
    qb = mx.quantize(wt.cuda(), block="2d")
    buf = torch.full((M + 40, N + 24), 7.0, dtype=torch.bfloat16, device="cuda")
    mx.gemm_fused_quant_a(ad, qb, out=buf[:M, :N])
    got = host(buf.float())
    assert np.all(got[M:] == 7.0) and np.all(got[:, N:] == 7.0), "wrote outside C"
    unfused = host(mx.gemm(mx.quantize(ad), qb, torch.bfloat16).float())
    assert np.array_equal(got[:M, :N], unfused)


def test_fused_quant_a_degenerate_shapes():
    """K = 0 writes zeros; M = 0 and N = 0 launch nothing; rows of A that are
    all zeros or hold a NaN give zero / NaN rows."""
    need_gpu()
    banner("fused quant A degenerate shapes")
    qb0 = mx.empty_mx(300, 0)
    c = torch.full((260, 300), 3.0, device="cuda")
    mx.gemm_fused_quant_a(torch.empty((260, 0), dtype=torch.bfloat16, device="cuda"), qb0, out=c)
    assert torch.count_nonzero(c).item() == 0
    qb = mx.quantize(torch.ones((300, 64), dtype=torch.bfloat16, device="cuda"))
    e = torch.empty((0, 300), device="cuda")
    mx.gemm_fused_quant_a(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), qb, out=e)
    a = torch.ones((260, 64), dtype=torch.bfloat16)
    a[5] = 0
    a[9, 40] = float("nan")
    c = host(mx.gemm_fused_quant_a(a.cuda(), qb))
    assert np.all(c[5] == 0) and np.isnan(c[9]).all()
    assert np.all(c[0] == 64.0)


def test_fused_quant_a_full_size_dgrad_sample():
    """The dgrad product at full size, dY 16384 x 5760 bf16 (the step's
    dY recipe, N(0, 1e-3)) times the transposed weight 2880 x 5760: equal bit
    for bit to mx_quantize + mx_gemm (an unsplit shape) everywhere, and to the
    oracle on 64 sampled rows."""
    need_gpu()
    M, N, K = 16384, 2880, 5760
    assert not _splits(M, N, K)
    g = torch.Generator().manual_seed(5)
    dy = (torch.randn((M, K), generator=g) * 1e-3).to(torch.bfloat16)
    w = torch.randn((N, K), generator=g).to(torch.bfloat16)
    banner("fused quant A full-size dgrad")
    dyd = dy.cuda()
    qw = mx.quantize(w.cuda(), block="2d")
    c = mx.gemm_fused_quant_a(dyd, qw, torch.bfloat16)
    unfused = mx.gemm(mx.quantize(dyd), qw, torch.bfloat16)
    assert torch.equal(c.view(torch.int16), unfused.view(torch.int16))
    rows = np.sort(np.random.default_rng(2).choice(M, 64, replace=False))
    ac, as_ = oracle.quantize(dy.float().numpy()[rows])
    bc, bs = oracle.quantize(w.float().numpy(), block="2d")
    ref, bound = oracle.gemm_ref(ac, as_, bc, bs, "1d", "2d")
    check_gemm(host(c.float())[rows], ref, bound, bf16=True, what="fused quant A dgrad")
