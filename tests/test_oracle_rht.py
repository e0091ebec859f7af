"""Pins for the 16-point random Hadamard transform: Sylvester structure
(scipy's Hadamard matrix), orthogonality, sign handling, axis semantics, and
the Wgrad identity (R dY)^T (R X) = dY^T X."""
import numpy as np
import pytest
import scipy.linalg

import oracle as O


def _matrix_of(signs):
    """The transform as a matrix, column j = transform of the unit vector e_j."""
    E = np.eye(16, dtype=np.float32)
    return O.rht16(E, axis=1, signs=signs).T.astype(np.float64)


def test_unsigned_transform_is_sylvester_hadamard_over_4():
    T = _matrix_of(0)
    H = scipy.linalg.hadamard(16)
    assert np.array_equal(T * 4, H)
    assert np.array_equal(H @ H.T, 16 * np.eye(16))


@pytest.mark.parametrize("signs", [0x0001, 0x8000, 0xE8D5, 0xFFFF, 0x1234])
def test_signed_transform_is_orthonormal(signs):
    T = _matrix_of(signs)
    D = np.diag([-1.0 if (signs >> i) & 1 else 1.0 for i in range(16)])
    assert np.array_equal(T, 0.25 * scipy.linalg.hadamard(16) @ D)
    assert np.allclose(T.T @ T, np.eye(16), atol=0, rtol=0)


def test_one_hot_gives_quarter_patterns():
    for j in range(16):
        e = np.zeros((1, 16), np.float32)
        e[0, j] = 1.0
        y = O.rht16(e, axis=1, signs=0)
        assert np.all(np.abs(y) == 0.25)


def test_axis_semantics():
    g = np.random.default_rng(0)
    x = g.standard_normal((32, 48)).astype(np.float32)
    s = 0xE8D5
    y0 = O.rht16(x, axis=0, signs=s)
    y1 = O.rht16(np.ascontiguousarray(x.T), axis=1, signs=s)
    assert np.array_equal(y0, y1.T)
    T = _matrix_of(s)
    ref = np.einsum("ij,cjn->cin", T, x.astype(np.float64).reshape(2, 16, 48)).reshape(32, 48)
    assert np.max(np.abs(y0 - ref)) <= 4e-7 * np.max(np.abs(x)) * 4


def test_wgrad_identity():
    """The transform is orthogonal along tokens, so (R dY)^T (R X) equals
    dY^T X up to fp32 rounding of the transformed operands."""
    g = np.random.default_rng(1)
    M, N, K = 64, 24, 40
    dy = g.standard_normal((M, N)).astype(np.float32)
    x = g.standard_normal((M, K)).astype(np.float32)
    s = O.rht_signs_from_seed(0)
    rdy = O.rht16(dy, axis=0, signs=s).astype(np.float64)
    rx = O.rht16(x, axis=0, signs=s).astype(np.float64)
    ref = dy.astype(np.float64).T @ x.astype(np.float64)
    got = rdy.T @ rx
    scale = np.abs(dy.astype(np.float64)).T @ np.abs(x.astype(np.float64))
    assert np.max(np.abs(got - ref) / scale) < 1e-6


def test_rht_inside_quantize_matches_standalone():
    """quantize(transpose, rht) uses the same transform as rht16 along axis 0:
    quantising the standalone output (no RHT) gives identical bytes."""
    g = np.random.default_rng(2)
    x = g.standard_normal((48, 32)).astype(np.float32)
    s = 0xE8D5
    q1 = O.quantize(x, transpose=True, rht=True, signs=s)
    y = O.rht16(x, axis=0, signs=s)
    q2 = O.quantize(np.ascontiguousarray(y.T))
    assert np.array_equal(q1.codes, q2.codes) and np.array_equal(q1.scales, q2.scales)
    assert q1.g == q2.g
