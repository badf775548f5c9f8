"""Whole output tiles of the full-size GEMM workloads against the oracle.

The other full-size tests sample rows and 32-column groups.  Here whole
256 x 256 output tiles (one workgroup's tile of the 256 x 256 kernels) and the
ragged tile at the N edge are compared element by element: fprop (N = 5760,
the edge tile holds columns 5632 .. 5759), the MoE grouped GEMM in its largest
expert (a row tile inside it) and its smallest (all its rows, a partial row
tile included), and dgrad (N = 2880, edge columns 2816 .. 2879).  The rule is
the GEMM rule of the other tests: |C - ref| <= 1e-5 * sum_k |a_k b_k| plus
half a bf16 ulp, ref the float64 product of the oracle's quantization of the
same input rows and weight columns ("MXFP4", AI Wiki, §Conversion rules).
"""
import numpy as np
import pytest
import torch

import mxfp4_microscaling_quantization_mx_amd as mx
import oracle
import workloads
from gpu_util import banner, check_gemm, host, need_gpu, to_dev

pytestmark = pytest.mark.gpu


def _tile_checks(got, rows, col_sets, quant_rows, quant_cols, what):
    """got: the GPU output (host); for each column set, quantize the weight
    columns with quant_cols and compare got[rows][:, cols]."""
    ac, as_ = quant_rows(rows)
    worst = 0.0
    for cols in col_sets:
        bc, bs, b_block = quant_cols(cols)
        ref, bound = oracle.gemm_ref(ac, as_, bc, bs, "1d", b_block)
        worst = max(worst, check_gemm(got[np.ix_(rows, cols)], ref, bound, bf16=True,
                                      what=f"{what} cols {cols[0]}..{cols[-1]}"))
    return worst


def test_fprop_whole_tiles():
    """X 16384x2880 (transform, RNE) times W 2880x5760 (32x32 tiles along dim 0,
    the same transform): rows 4096..4351 against the interior tile of columns
    2560..2815 and the edge tile 5632..5759."""
    need_gpu()
    x, w = workloads.fprop()
    mask = workloads.rht_mask(workloads.CFG_FPROP)
    banner("fprop whole tiles")
    qx = mx.quantize(x.cuda(), rht_mask=mask)
    qw = mx.quantize(w.cuda(), axis="dim0", block="2d", rht_mask=mask)
    y = host(mx.gemm(qx, qw, torch.bfloat16).float())
    xn, wn = x.float().numpy(), w.float().numpy()
    worst = _tile_checks(
        y, np.arange(4096, 4352), [np.arange(2560, 2816), np.arange(5632, 5760)],
        lambda r: oracle.quantize(xn[r], rht_mask=mask),
        lambda c: (*oracle.quantize(wn[:, c], axis="dim0", block="2d", rht_mask=mask), "2d"), "fprop")
    print(f"fprop whole tiles: max |err| / sum|ab| = {worst:.2e}")


def test_dgrad_whole_tiles():
    """dY 16384x5760 (stochastic rounding along its last dim) times the forward
    weight transposed on the GPU (2880 x 5760 in 32x32 tiles): rows
    8192..8447 against the interior tile of columns 1024..1279 and the edge
    tile 2816..2879."""
    need_gpu()
    dy, w = workloads.dgrad()
    seed = workloads.philox_seed(workloads.CFG_DGRAD)
    banner("dgrad whole tiles")
    qwt = mx.transpose(mx.quantize(w.cuda(), axis="dim0", block="2d"))
    qd = mx.quantize(dy.cuda(), rounding="sr", seed=seed)
    dx = host(mx.gemm(qd, qwt, torch.bfloat16).float())
    dyn, wn = dy.float().numpy(), w.float().numpy()

    def quant_w(cols):
        c, s = oracle.quantize(wn[cols], axis="dim0", block="2d")      # tiles of W^T: [5760, len] blocked along 5760
        c, s = oracle.transpose_2d(c, s)
        return c, s, "2d"

    worst = _tile_checks(
        dx, np.arange(8192, 8448), [np.arange(1024, 1280), np.arange(2816, 2880)],
        lambda r: oracle.quantize(dyn[r], rounding="sr", seed=seed, row_index=r, K_total=5760), quant_w, "dgrad")
    print(f"dgrad whole tiles: max |err| / sum|ab| = {worst:.2e}")


def test_moe_whole_tiles():
    """MoE grouped GEMM (32 experts, 16384 tokens x top-4 by Zipf 1.1): a whole
    row tile in the middle of the largest expert and every row of the smallest
    expert, each against an interior column tile and the edge tile of columns
    5632..5759 of its own expert's weight."""
    need_gpu()
    tok, offsets = workloads.moe_routing()
    E, K, N = 32, 2880, 5760
    banner("moe whole tiles: quantize")
    xc = workloads.to_bf16(workloads.moe_tokens())
    qa = mx.quantize_gather(xc.cuda(), torch.from_numpy(tok.astype(np.int32)).cuda())
    qb = mx.empty_mx(N, K, "2d", experts=E)
    for e in range(E):
        mx.quantize(workloads.to_bf16(workloads.moe_expert_weight(e)).cuda(), axis="dim0", block="2d",
                    out=mx.expert(qb, e))
    banner("moe whole tiles: grouped gemm")
    y = host(mx.grouped_gemm(qa, to_dev(np.asarray(offsets, dtype=np.int32)), qb, torch.bfloat16).float())
    xn = xc.float().numpy()
    sizes = np.diff(offsets)
    big, small = int(np.argmax(sizes)), int(np.argmin(sizes))
    lo = int(offsets[big])
    mid = lo + (sizes[big] // 2 // 256) * 256
    worst = 0.0
    for e, rows in [(big, np.arange(mid, mid + 256)), (small, np.arange(offsets[small], offsets[small + 1]))]:
        wn = workloads.to_bf16(workloads.moe_expert_weight(e)).float().numpy()
        worst = max(worst, _tile_checks(
            y, rows, [np.arange(1280, 1536), np.arange(5632, 5760)],
            lambda r: oracle.quantize(xn[tok[r]]),
            lambda c: (*oracle.quantize(wn[:, c], axis="dim0", block="2d"), "2d"), f"moe expert {e}"))
    print(f"moe whole tiles (experts {big}: {sizes[big]} rows, {small}: {sizes[small]} rows): "
          f"max |err| / sum|ab| = {worst:.2e}")


@pytest.mark.parametrize("elem", ["e4m3", "e2m3"])
def test_fprop_mxfp8_mxfp6_whole_tiles(elem):
    """The fprop shape with MXFP8 (E4M3) or MXFP6 (E2M3) operands, quantized
    on the GPU (X along its last dim, W along dim 0, RNE): rows 4096..4351
    against the interior tile of columns 2560..2815 and the edge tile
    5632..5759, within the float32 bound plus the scaled MFMA's
    internal-precision allowance for FP8/FP6 operands and half a bf16 ulp."""
    need_gpu()
    from gpu_util import bf16_half_ulp, mx_group_bound
    x, w = workloads.fprop()
    banner(f"fprop {elem} whole tiles")
    qx = mx.quantize(x.cuda(), elem=elem)
    qw = mx.quantize(w.cuda(), axis="dim0", elem=elem)
    y = host(mx.gemm(qx, qw, torch.bfloat16).float()).astype(np.float64)
    xn, wn = x.float().numpy(), w.float().numpy()
    rows = np.arange(4096, 4352)
    ac, as_ = oracle.quantize(xn[rows], elem=elem)
    av = oracle.gemm.dequant_f64(ac, as_, elem)
    for cols in (np.arange(2560, 2816), np.arange(5632, 5760)):
        bc, bs = oracle.quantize(wn[:, cols], axis="dim0", elem=elem)
        ref, bound = oracle.gemm_ref(ac, as_, bc, bs, a_elem=elem, b_elem=elem)
        got = y[np.ix_(rows, cols)]
        tol = 1e-5 * bound + mx_group_bound(av, oracle.gemm.dequant_f64(bc, bs, elem))
        tol = tol + bf16_half_ulp(np.maximum(np.abs(got), np.abs(ref)))
        assert np.all(np.abs(got - ref) <= tol), f"{elem} cols {cols[0]}..{cols[-1]}"
