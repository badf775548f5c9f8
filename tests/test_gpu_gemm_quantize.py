"""GPU parity of mx_gemm_quantize, the GEMM whose epilogue quantizes the
product along N into MXFP4 (1-D blocks, RNE) instead of storing it.

Three checks per case:
* bit-exact against the unfused composition on the same device: mx_gemm with
  float32 output (the same MFMA accumulation, so the same float32 values)
  followed by mx_quantize of that output along its last dim;
* bit-exact against the oracle's quantize of that float32 product (every
  rounding decision in float32 on both sides);
* the float32 product itself against the oracle's float64 GEMM reference
  within the GEMM bound, so the composition is anchored to the pages'
  arithmetic end to end.
Padding bytes of the output rows are filled with a marker and must survive.
"""
import numpy as np
import pytest
import torch

import mxfp4_microscaling_quantization_mx_amd as mx
import oracle
import workloads
from gpu_util import banner, check_gemm, codes_equal, host, need_gpu
from test_gpu_gemm import _rand_mx, _upload

pytestmark = pytest.mark.gpu


def _full_rows(t):
    return t.as_strided((t.shape[0], t.stride(0)), (t.stride(0), 1))


def _marked_out(M, N, fill=0x5A):
    q = mx.empty_mx(M, N)
    _full_rows(q.codes).fill_(fill)
    _full_rows(q.scales).fill_(fill)
    return q


def _check_fused(a, b, M, N, scale_mode, ref_inputs=None):
    fused = _marked_out(M, N)
    mx.gemm_quantize(a, b, scale_mode=scale_mode, out=fused)
    y = mx.gemm(a, b, torch.float32)
    unfused = mx.quantize(y, scale_mode=scale_mode)
    fc, fs = host(fused.codes), host(fused.scales)
    codes_equal(fc, host(unfused.codes), "codes vs gemm + quantize")
    codes_equal(fs, host(unfused.scales), "scales vs gemm + quantize")
    yn = host(y)
    oc, os_ = oracle.quantize(yn, scale_mode=scale_mode)
    codes_equal(fc, oc, "codes vs oracle quantize of the product")
    codes_equal(fs, os_, "scales vs oracle quantize of the product")
    assert np.all(host(_full_rows(fused.codes))[:, N // 2:] == 0x5A), "code row padding written"
    assert np.all(host(_full_rows(fused.scales))[:, N // 32:] == 0x5A), "scale row padding written"
    if ref_inputs is not None:
        ref, bound = oracle.gemm_ref(*ref_inputs)
        check_gemm(yn, ref, bound, what="product")
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
    48 sampled rows equal the oracle's quantize of those rows of the product."""
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
    rows = np.sort(np.random.default_rng(4).choice(16384, 48, replace=False))
    oc, os_ = oracle.quantize(host(y)[rows])
    codes_equal(host(fused.codes)[rows], oc, "sampled rows vs oracle")
    codes_equal(host(fused.scales)[rows], os_, "sampled scales vs oracle")
