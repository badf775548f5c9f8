"""Pins for the oracle's format layer against the page's tables.

"MXFP4", AI Wiki, §Format specification: parameter table and E2M1 value table.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.formats import BLOCK
from golden_io import e2m1_table, params


def test_e2m1_decode_matches_page_table():
    table = e2m1_table()
    assert len(table) == 8
    for code, value, _ in table:
        assert oracle.e2m1_decode(code) == value
        # negative half: same pattern with the sign bit set
        neg = oracle.e2m1_decode(code | 0b1000)
        assert neg == -value
        assert math.copysign(1.0, neg) == -1.0      # -0 keeps its sign


def test_e2m1_grid_and_range_from_params():
    p = params("mxfp4_params.txt")
    grid = oracle.E2M1_GRID
    assert list(grid) == [v for _, v, _ in e2m1_table()]
    assert grid.max() == float(p["e2m1_max_normal"])
    assert min(v for c, v, k in e2m1_table() if k == "normal") == float(p["e2m1_min_normal"])
    assert min(v for c, v, k in e2m1_table() if k == "subnormal") == float(p["e2m1_subnormal"])
    # no Inf / NaN encodings among the 16 codes
    allv = oracle.e2m1_decode(np.arange(16))
    assert np.isfinite(allv).all()


def test_e8m0_decode_from_params():
    p = params("mxfp4_params.txt")
    bias = int(p["e8m0_bias"])
    nan_code = int(p["e8m0_nan_code"], 2)
    codes = np.arange(256)
    v = oracle.e8m0_decode(codes)
    assert np.isnan(v[nan_code]) and np.isnan(v).sum() == 1
    finite = v[:nan_code]
    # power-of-two only, strictly doubling, no zero, no infinity
    assert (finite > 0).all() and np.isfinite(finite).all()
    assert np.all(finite[1:] == 2 * finite[:-1])
    assert finite[bias] == 1.0
    assert finite[0] == 2.0 ** int(p["e8m0_min_exponent"])
    assert finite[-1] == 2.0 ** int(p["e8m0_max_exponent"])


def test_bits_per_block_from_quantized_sizes():
    p = params("mxfp4_params.txt")
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 32 * 9)).astype(np.float32)
    codes, scales = oracle.quantize(x)
    nblocks = x.size // BLOCK
    bits = (codes.nbytes + scales.nbytes) * 8
    assert bits == nblocks * int(p["bits_per_block"])
    assert bits / x.size == float(p["bits_per_value"])
    assert int(p["block_size"]) == BLOCK


def test_nan_scale_poisons_block():
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, :] = 0x53                               # arbitrary non-zero nibbles
    scales = np.array([[127, 0xFF]], dtype=np.uint8)
    out = oracle.dequantize(codes, scales)
    assert np.isfinite(out[0, :32]).all()
    assert np.isnan(out[0, 32:]).all()


def test_bf16_widening_exact():
    bits = np.array([0x3F80, 0xBF80, 0x7F80, 0x0001, 0x4049], dtype=np.uint16)
    f = oracle.bf16_bits_to_f32(bits)
    assert f[0] == 1.0 and f[1] == -1.0 and np.isinf(f[2])
    assert f[3] == np.float32(2.0 ** -133)
    assert f[4] == np.float32(3.140625)
