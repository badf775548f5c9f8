"""Pins for the oracle GEMM reference.

"MXFP4", AI Wiki, §Conversion rules: a block dot product is
X(A) X(B) sum_i P_i(A) P_i(B) and a long dot product is the sum of block dot
products.  The float64 BLAS reference is checked against that definition
evaluated in exact rational arithmetic (brute force, small sizes), including
2-D scale broadcasting, NaN scales, and the grouped (per-expert) variant.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.quantize import unpack_nibbles


def _rand_operand(rng, rows, k, block="1d", lo=124, hi=131):
    codes = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    srows = rows // 32 if block == "2d" else rows
    scales = rng.integers(lo, hi, size=(srows, k // 32), dtype=np.uint8)
    return codes, scales


def _exact_gemm(ac, asc, bc, bsc, a_block="1d", b_block="1d"):
    a = unpack_nibbles(ac)
    b = unpack_nibbles(bc)
    M, K = a.shape
    N = b.shape[0]
    out = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for kb in range(K // 32):
                sa = asc[m // 32 if a_block == "2d" else m, kb]
                sb = bsc[n // 32 if b_block == "2d" else n, kb]
                tot += oracle.block_dot_exact(a[m, kb * 32:(kb + 1) * 32], sa,
                                              b[n, kb * 32:(kb + 1) * 32], sb)
            out[m, n] = tot
    return out


@pytest.mark.parametrize("a_block,b_block", [("1d", "1d"), ("1d", "2d"), ("2d", "2d")])
def test_gemm_ref_matches_exact_rational(a_block, b_block):
    rng = np.random.default_rng(21)
    M, N, K = 32, 32, 96
    ac, asc = _rand_operand(rng, M, K, a_block)
    bc, bsc = _rand_operand(rng, N, K, b_block)
    ref, bound = oracle.gemm_ref(ac, asc, bc, bsc, a_block, b_block)
    exact = _exact_gemm(ac, asc, bc, bsc, a_block, b_block)
    # scales within 2^+-4: every partial sum is a multiple of 2^-10 below 2^30,
    # so the float64 reference is exact
    for m in range(0, M, 3):
        for n in range(0, N, 5):
            assert Fraction(ref[m, n]) == exact[m, n]
    assert np.all(bound >= np.abs(ref))


def test_gemm_ref_wide_scales_within_float64_bound():
    rng = np.random.default_rng(22)
    M, N, K = 8, 8, 128
    ac, asc = _rand_operand(rng, M, K, lo=60, hi=200)
    bc, bsc = _rand_operand(rng, N, K, lo=60, hi=200)
    ref, bound = oracle.gemm_ref(ac, asc, bc, bsc)
    exact = _exact_gemm(ac, asc, bc, bsc)
    for m in range(M):
        for n in range(N):
            err = abs(Fraction(ref[m, n]) - exact[m, n])
            assert err <= Fraction(K * 2.0 ** -52) * Fraction(bound[m, n])


def test_single_block_exact_and_identity_probe():
    """K = 32: one code per row set to 1.0 picks out single products."""
    ac = np.zeros((32, 16), np.uint8)
    bc = np.zeros((32, 16), np.uint8)
    for i in range(32):
        j = i // 2
        ac[i, j] = 0x2 << (4 * (i % 2))      # code 2 = 1.0 at element i
    rng = np.random.default_rng(3)
    bc = rng.integers(0, 256, size=(32, 16), dtype=np.uint8)
    asc = np.full((32, 1), 127, np.uint8)
    bsc = rng.integers(120, 135, size=(32, 1), dtype=np.uint8)
    ref, _ = oracle.gemm_ref(ac, asc, bc, bsc)
    b = oracle.dequantize(bc, bsc).astype(np.float64)
    assert np.array_equal(ref, b.T)          # row i of A is e_i


def test_nan_scale_poisons_outputs():
    rng = np.random.default_rng(4)
    ac, asc = _rand_operand(rng, 4, 64)
    bc, bsc = _rand_operand(rng, 3, 64)
    asc[2, 1] = 0xFF
    bsc[0, 0] = 0xFF
    ref, _ = oracle.gemm_ref(ac, asc, bc, bsc)
    assert np.isnan(ref[2, :]).all() and np.isnan(ref[:, 0]).all()
    assert np.isfinite(ref[[0, 1, 3]][:, [1, 2]]).all()


def test_sampled_rows_cols_match_full():
    rng = np.random.default_rng(5)
    ac, asc = _rand_operand(rng, 64, 128, "2d")
    bc, bsc = _rand_operand(rng, 96, 128, "2d")
    full, fb = oracle.gemm_ref(ac, asc, bc, bsc, "2d", "2d")
    rows = np.array([63, 0, 33, 5])
    cols = np.array([95, 1, 40])
    part, pb = oracle.gemm_ref(ac, asc, bc, bsc, "2d", "2d", rows=rows, cols=cols)
    assert np.array_equal(part, full[np.ix_(rows, cols)])
    assert np.array_equal(pb, fb[np.ix_(rows, cols)])


def test_grouped_ref_matches_per_expert_exact():
    rng = np.random.default_rng(6)
    E, N, K = 4, 32, 64
    offsets = np.array([0, 5, 5, 37, 40])        # an empty expert and ragged sizes
    M = offsets[-1]
    ac, asc = _rand_operand(rng, M, K)
    bcs, bss = [], []
    for _ in range(E):
        c, s = _rand_operand(rng, N, K, "2d")
        bcs.append(c)
        bss.append(s)
    bc, bs = np.stack(bcs), np.stack(bss)
    ref, _ = oracle.grouped_gemm_ref(ac, asc, offsets, bc, bs)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        ex = _exact_gemm(ac[lo:hi], asc[lo:hi], bc[e], bs[e], "1d", "2d")
        for i in range(hi - lo):
            for n in range(0, N, 7):
                assert Fraction(ref[lo + i, n]) == ex[i, n]


def test_quantized_gemm_approximates_float_gemm():
    """Sanity: the dequantized product tracks the unquantized one (RHT on both
    operands with one mask cancels: H^T H = I up to the rounding of c)."""
    rng = np.random.default_rng(7)
    a = rng.standard_normal((64, 256)).astype(np.float32)
    b = rng.standard_normal((48, 256)).astype(np.float32)
    exact = a.astype(np.float64) @ b.astype(np.float64).T
    for mask in (None, 0x5A5AA5A5):
        ac, asc = oracle.quantize(a, rht_mask=mask)
        bc, bsc = oracle.quantize(b, rht_mask=mask)
        ref, _ = oracle.gemm_ref(ac, asc, bc, bsc)
        rel = np.linalg.norm(ref - exact) / np.linalg.norm(exact)
        assert rel < 0.25        # MXFP4 noise on both operands (~0.11 relative each)


def test_quantized_product_check_accepts_the_oracle_and_rejects_one_bit_errors():
    """The GPU tests check fused GEMM+quantize outputs with
    gpu_util.check_quantized_product (the oracle's quantization of the float64
    product within the float32 accumulation error).  On the CPU: the oracle's
    own quantization of the product passes in every scale mode, and a single
    flipped code bit or a scale byte one too large fails."""
    import sys, os
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from gpu_util import check_quantized_product
    rng = np.random.default_rng(0)
    ac = rng.integers(0, 256, (48, 1440), dtype=np.uint8)
    as_ = rng.integers(120, 135, (48, 90), dtype=np.uint8)
    bc = rng.integers(0, 256, (64, 1440), dtype=np.uint8)
    bs = rng.integers(120, 135, (64, 90), dtype=np.uint8)
    ref, S = oracle.gemm_ref(ac, as_, bc, bs)
    for mode in ("floor", "round_up", "prescale_3_4"):
        qc, qs = oracle.quantize(ref.astype(np.float32), scale_mode=mode)
        check_quantized_product(qc, qs, ref, S, 2880, mode)
        bad = qc.copy()
        bad[3, 5] ^= 0x01
        with pytest.raises(AssertionError):
            check_quantized_product(bad, qs, ref, S, 2880, mode)
        bads = qs.copy()
        bads[2, 1] += 1
        with pytest.raises(AssertionError):
            check_quantized_product(qc, bads, ref, S, 2880, mode)
