"""Pins for the oracle's 32-point randomized Hadamard transform.

The pages name the transform and its size (32 for MXFP4: "MXFP4", AI Wiki,
§Training with MXFP4).  Pins: SciPy's Hadamard matrix (an independent library
routine), H H^T = 32 I, the float32 fast transform against a float64 matrix
product, orthonormality (norm preservation, round trip) and the sign mask.
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle.rht import RHT_C


def test_hadamard_matches_scipy_and_is_orthogonal():
    h = oracle.hadamard32_f64()
    assert np.array_equal(h, scipy.linalg.hadamard(32).astype(np.float64))
    assert np.array_equal(h @ h.T, 32 * np.eye(32))


def test_normalisation_constant():
    assert np.float32(RHT_C) == np.float32(1.0 / np.sqrt(32.0))
    assert np.array([RHT_C], np.float32).view(np.uint32)[0] == 0x3E3504F3


@pytest.mark.parametrize("mask", [0, 0xFFFFFFFF, 0x12345678, 0x80000001])
def test_fast_transform_matches_matrix_product(mask):
    rng = np.random.default_rng(mask & 0xFFFF)
    x = rng.standard_normal((500, 32)).astype(np.float32)
    y = oracle.rht_forward_f32(x, mask).astype(np.float64)
    d = np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(32)])
    ref = (scipy.linalg.hadamard(32) @ (x.astype(np.float64) * d).T).T / np.sqrt(32.0)
    # five float32 add stages + one multiply: relative to the block's 2-norm
    err = np.abs(y - ref).max(axis=1) / np.linalg.norm(x.astype(np.float64), axis=1)
    assert err.max() < 8 * 2.0 ** -24 * np.sqrt(32)


def test_norm_preserved_and_round_trip():
    rng = np.random.default_rng(11)
    x = rng.standard_t(3, (1000, 32)).astype(np.float32)
    mask = 0xDEADBEEF
    y = oracle.rht_forward_f32(x, mask)
    n0 = np.linalg.norm(x.astype(np.float64), axis=1)
    n1 = np.linalg.norm(y.astype(np.float64), axis=1)
    assert np.max(np.abs(n1 - n0) / n0) < 1e-6
    back = oracle.rht_inverse_f32(y, mask).astype(np.float64)
    assert np.max(np.linalg.norm(back - x, axis=1) / n0) <= 1e-6


def test_sign_mask_bit_i_negates_element_i():
    e = np.zeros((32, 32), dtype=np.float32)
    np.fill_diagonal(e, 1.0)
    base = oracle.rht_forward_f32(e, 0)
    for i in (0, 5, 31):
        flipped = oracle.rht_forward_f32(e, 1 << i)
        assert np.array_equal(flipped[i], -base[i])
        others = [j for j in range(32) if j != i]
        assert np.array_equal(flipped[others], base[others])


def test_impulse_gives_scaled_hadamard_row():
    """RHT of e_j (no signs) is c times column j of H (Sylvester order, no bit reversal)."""
    h = scipy.linalg.hadamard(32)
    for j in (0, 1, 6, 17):
        e = np.zeros((1, 32), dtype=np.float32)
        e[0, j] = 1.0
        y = oracle.rht_forward_f32(e, 0)[0]
        assert np.array_equal(y, (h[:, j] * RHT_C).astype(np.float32))
