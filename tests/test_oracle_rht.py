"""Pins for oracle.rht: the 16-wide random Hadamard transform.

Independent references: scipy.linalg.hadamard(16) (Sylvester order), exact
orthogonality in fp64, an fp32 error bound against the fp64 matrix product,
and cancellation of the transform inside a product (TetraJet-v2 technical
summary, section 2.C: the transform is applied to both operands of dX / dW).
"""
import numpy as np
import pytest
from scipy.linalg import hadamard

from oracle import rht


def test_matrix_is_sylvester_hadamard():
    np.testing.assert_array_equal(rht.rht_matrix_f64(0), hadamard(16) / 4.0)


@pytest.mark.parametrize("mask", [0, 1, 0x8000, 0xA5A5, 0xFFFF, 0x1234])
def test_orthogonal_exact(mask):
    T = rht.rht_matrix_f64(mask)
    np.testing.assert_array_equal(T.T @ T, np.eye(16))
    np.testing.assert_array_equal(T, (hadamard(16) / 4.0) @ np.diag(rht.sign_vector(mask)))


@pytest.mark.parametrize("mask", [0, 0xA5A5, 0x1234])
def test_fp32_butterfly_vs_fp64_matrix(mask):
    x = np.random.default_rng(mask).standard_normal((4096, 16)).astype(np.float32)
    x[::7] *= np.float32(1e3)
    y32 = rht.fwht16_f32(x, mask).astype(np.float64)
    y64 = x.astype(np.float64) @ rht.rht_matrix_f64(mask).T
    # 4 rounded add stages on partial sums bounded by the chunk's 1-norm, then an exact *0.25
    bound = 0.25 * 4 * 2.0 ** -24 * np.abs(x.astype(np.float64)).sum(axis=1, keepdims=True)
    assert np.all(np.abs(y32 - y64) <= bound)
    n32 = np.linalg.norm(y32, axis=1)
    n64 = np.linalg.norm(x.astype(np.float64), axis=1)
    np.testing.assert_allclose(n32, n64, rtol=4 * 2.0 ** -24 * 4)


def test_transform_cancels_in_product():
    r = np.random.default_rng(1)
    A = r.standard_normal((8, 64)).astype(np.float32)
    B = r.standard_normal((5, 64)).astype(np.float32)
    TA = rht.rht_along_last(A, 0x3C5A).astype(np.float64)
    TB = rht.rht_along_last(B, 0x3C5A).astype(np.float64)
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    np.testing.assert_allclose(TA @ TB.T, ref, rtol=0, atol=1e-4 * np.abs(ref).max())
    # a different mask on one side does not cancel
    TB2 = rht.rht_along_last(B, 0x3C5B).astype(np.float64)
    assert np.abs(TA @ TB2.T - ref).max() > 1e-2


@pytest.mark.parametrize("j", range(16))
def test_sign_bit_order_one_hot(j):
    """Bit j of the mask negates position j of each 16-chunk, i.e. column j of (1/4) H16: built
    from scipy's Hadamard matrix, so a reversed or shifted bit-to-position map fails."""
    ref = hadamard(16) / 4.0
    ref[:, j] = -ref[:, j]
    np.testing.assert_array_equal(rht.rht_matrix_f64(1 << j), ref)
    # the fp32 butterfly on small integers is exact: it must equal the scipy product
    x = np.arange(1, 17, dtype=np.float32) * np.float32(3.0) - np.float32(20.0)
    np.testing.assert_array_equal(rht.fwht16_f32(x, 1 << j).astype(np.float64), ref @ x.astype(np.float64))
