"""GPU parity of the split-K ("stream-K") form of mx_gemm.

Shapes with too few 256x256 output tiles for the chip (or a K too long for one
float32 accumulator) are cut along K into segments whose float32 partial
products are added in a fixed order ("MXFP4", AI Wiki, §Conversion rules: the long
dot product is a sum of block dot products accumulated in float32).  The rule
is the GEMM rule of the other tests: |C - ref| <= 1e-5 * sum_k |a_k b_k| per
output against the oracle's float64 product of the dequantized operands.  On
top of it: results are identical bit for bit from run to run (the summation
order does not depend on which workgroup finishes last), nothing outside C is
written, NaN scales propagate, and the full-size weight gradient is checked
on a whole interior tile and on the ragged edge tile.
"""
import numpy as np
import pytest
import torch

import mxfp4_microscaling_quantization_mx_amd as mx
import oracle
import workloads
from gpu_util import banner, check_gemm, host, need_gpu, to_dev
from test_gpu_gemm import _rand_mx, _upload

pytestmark = pytest.mark.gpu


def _splits(M, N, K):
    return mx.load_library().mx_gemm_workspace_size(M, N, K) > 0


@pytest.mark.parametrize("M,N,K,a_block,b_block", [
    (512, 512, 16384, "1d", "1d"),     # 4 tiles, long K: many segments per tile
    (300, 520, 4128, "1d", "1d"),      # ragged M and N, odd stage count (a padding stage), 1-block K tail
    (288, 288, 2880, "1d", "2d"),      # the fprop K with 2-D weight tiles
    (1024, 1024, 2880, "2d", "2d"),
    (520, 288, 6016, "1d", "2d"),      # 3-block K tail
])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_splitk_matches_oracle(M, N, K, a_block, b_block, out):
    need_gpu()
    assert _splits(M, N, K), "shape expected to be split along K"
    rng = np.random.default_rng(M + 5 * N + 11 * K)
    ac, as_ = _rand_mx(rng, M, K, a_block)
    bc, bs = _rand_mx(rng, N, K, b_block)
    banner(f"splitk M={M} N={N} K={K} {a_block}/{b_block} {out}")
    c = host(mx.gemm(_upload(ac, as_, a_block), _upload(bc, bs, b_block), out).float())
    ref, bound = oracle.gemm_ref(ac, as_, bc, bs, a_block, b_block)
    check_gemm(c, ref, bound, bf16=(out == torch.bfloat16), what="splitk")


def test_splitk_is_deterministic_and_leaves_workspace_reusable():
    """Three calls on the same workspace give the same bits (the tile sums are
    taken in segment order whatever the arrival order), and a different shape
    in between does not disturb it."""
    need_gpu()
    rng = np.random.default_rng(21)
    M, N, K = 768, 512, 8192
    ac, as_ = _rand_mx(rng, M, K)
    bc, bs = _rand_mx(rng, N, K)
    a, b = _upload(ac, as_), _upload(bc, bs)
    banner("splitk determinism")
    first = host(mx.gemm(a, b, torch.float32))
    xc, xs = _rand_mx(rng, 300, 4128)
    mx.gemm(_upload(xc, xs), _upload(xc, xs), torch.float32)
    for _ in range(2):
        again = host(mx.gemm(a, b, torch.float32))
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
    ref, bound = oracle.gemm_ref(ac, as_, bc, bs)
    check_gemm(first, ref, bound, what="splitk determinism")


def test_splitk_workspace_shared_by_shapes_with_more_tiles():
    """A workspace first used by a 4-tile shape (whose partials land right
    after the counters) and then by an 81-tile one: the second call must find
    its tile counters at zero, not the first call's partials."""
    need_gpu()
    rng = np.random.default_rng(24)
    ws = torch.zeros(max(mx.load_library().mx_gemm_workspace_size(*s) for s in [(512, 512, 16384),
                                                                                (2304, 2304, 4096)]),
                     dtype=torch.uint8, device="cuda")
    ac, as_ = _rand_mx(rng, 512, 16384)
    mx.gemm(_upload(ac, as_), _upload(ac, as_), torch.float32, workspace=ws)
    M = N = 2304
    K = 4096
    assert _splits(M, N, K)
    ac, as_ = _rand_mx(rng, M, K)
    bc, bs = _rand_mx(rng, N, K)
    banner("splitk shared workspace")
    for _ in range(2):
        c = host(mx.gemm(_upload(ac, as_), _upload(bc, bs), torch.float32, workspace=ws))
        rows = np.arange(0, M, 37)
        ref, bound = oracle.gemm_ref(ac[rows], as_[rows], bc, bs)
        check_gemm(c[rows], ref, bound, what="splitk shared workspace")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_splitk_writes_nothing_outside_c(out_dtype):
    need_gpu()
    rng = np.random.default_rng(22)
    M, N, K = 300, 520, 4128
    ac, as_ = _rand_mx(rng, M, K)
    bc, bs = _rand_mx(rng, N, K)
    buf = torch.full((M + 50, N + 24), 7.0, dtype=out_dtype, device="cuda")
    banner(f"splitk guard rows {out_dtype}")
    mx.gemm(_upload(ac, as_), _upload(bc, bs), out=buf[:M, :N])
    c = host(buf.float())
    assert np.all(c[M:] == 7.0) and np.all(c[:, N:] == 7.0), "wrote outside C"
    ref, bound = oracle.gemm_ref(ac, as_, bc, bs)
    check_gemm(c[:M, :N], ref, bound, bf16=(out_dtype == torch.bfloat16), what="splitk guarded")


def test_splitk_nan_scale_propagates():
    """A NaN scale in any K segment poisons its outputs through the partial
    sums ("MXFP4", AI Wiki, §Format specification)."""
    need_gpu()
    rng = np.random.default_rng(23)
    M, N, K = 512, 512, 16384
    ac, as_ = _rand_mx(rng, M, K)
    bc, bs = _rand_mx(rng, N, K)
    as_[7, 3] = 0xFF          # early segment
    bs[300, 500] = 0xFF       # late segment
    banner("splitk nan")
    c = host(mx.gemm(_upload(ac, as_), _upload(bc, bs), torch.float32))
    ref, bound = oracle.gemm_ref(ac, as_, bc, bs)
    check_gemm(c, ref, bound, what="splitk nan")
    assert np.isnan(c[7]).all() and np.isnan(c[:, 300]).all()


def test_mfma_fp4_step_adds_exact_sum_with_one_rounding():
    """The accumulation model behind the split-K error bound: one 64-deep FP4
    step adds the exact sum of its products (two blocks with scales 2^0 and
    2^-20 here) to the float32 accumulator with a single rounding.  Step 1
    contributes +1152, step 2 contributes -1152 + 2^-22 (block 2: 32 x 6 x -6;
    block 3: 0.5 x 0.5 x 2^-20), so the exact result 2^-22 survives only if the
    step's internal sum is not rounded before it reaches the accumulator."""
    need_gpu()
    M = N = 256
    K = 128
    ac = np.zeros((M, K // 2), np.uint8)
    bc = np.zeros((N, K // 2), np.uint8)
    as_ = np.full((M, K // 32), 127, np.uint8)
    bs = np.full((N, K // 32), 127, np.uint8)
    ac[0, 0:16] = 0x77        # block 0: +6
    bc[0, 0:16] = 0x77
    ac[0, 32:48] = 0x77       # block 2: +6
    bc[0, 32:48] = 0xFF       # block 2: -6
    ac[0, 48] = 0x01          # block 3, element 0: 0.5
    bc[0, 48] = 0x01
    as_[0, 3] = bs[0, 3] = 117  # 2^-10 each
    banner("mfma single rounding probe")
    c = host(mx.gemm(_upload(ac, as_), _upload(bc, bs), torch.float32))
    ref, _ = oracle.gemm_ref(ac, as_, bc, bs)
    assert ref[0, 0] == 2.0 ** -22
    print(f"probe result {c[0, 0]!r} (exact 2^-22 = {2.0 ** -22!r})")
    assert c[0, 0] == np.float32(2.0 ** -22)
    assert np.all(c[1:] == 0) and np.all(c[0, 1:] == 0)


def test_wgrad_full_size_whole_tiles():
    """The weight-gradient workload (dY N(0,1e-3), X N(0,1), 16384 x 2880 bf16,
    both quantized along the 16384 token dim with the transform and stochastic
    rounding; dW 2880 x 2880 float32, split along K): one whole interior
    256 x 256 output tile and the ragged corner tile (rows and columns
    2816 .. 2879) element by element against the oracle."""
    need_gpu()
    assert _splits(2880, 2880, 16384)
    dy, x = workloads.wgrad()
    mask = workloads.rht_mask(workloads.CFG_WGRAD)
    seed = workloads.philox_seed(workloads.CFG_WGRAD)
    banner("wgrad full size whole tiles")
    qd = mx.quantize(dy.cuda(), axis="dim0", rht_mask=mask, rounding="sr", seed=seed, offset=0)
    qx = mx.quantize(x.cuda(), axis="dim0", rht_mask=mask, rounding="sr", seed=seed, offset=1)
    dw = host(mx.gemm(qd, qx, torch.float32))
    dyn, xn = dy.float().numpy(), x.float().numpy()
    worst = 0.0
    for rows, cols in [(np.arange(1280, 1536), np.arange(768, 1024)), (np.arange(2816, 2880), np.arange(2816, 2880)),
                       (np.arange(2816, 2880), np.arange(0, 256))]:
        odc, ods = oracle.quantize(dyn[:, rows], axis="dim0", rht_mask=mask, rounding="sr", seed=seed,
                                   offset=0, row_index=rows)
        oxc, oxs = oracle.quantize(xn[:, cols], axis="dim0", rht_mask=mask, rounding="sr", seed=seed,
                                   offset=1, row_index=cols)
        ref, bound = oracle.gemm_ref(odc, ods, oxc, oxs)
        worst = max(worst, check_gemm(dw[np.ix_(rows, cols)], ref, bound, what="wgrad tile"))
    print(f"wgrad whole tiles: max |err| / sum|ab| = {worst:.3e}")
