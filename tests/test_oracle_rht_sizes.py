"""Pins of the oracle's Hadamard transforms of size 4, 16 and 128 [Review s3
and its size note; Captions Fig. 12] and of the sign options [Captions
Fig. 13: no randomisation, one fixed seed, a seed per layer] (CPU only)."""
import numpy as np
import pytest
from scipy.linalg import hadamard

import oracle as O


def _bits(signs, d):
    return np.array([(int(signs[i // 32]) >> (i % 32)) & 1 for i in range(d)])


@pytest.mark.parametrize("d", [4, 16, 128])
@pytest.mark.parametrize("seed", [0, 7, 2 ** 40 + 3])
def test_matches_scipy_sylvester_matrix(d, seed):
    """y = H_d diag(s) x / sqrt(d) with scipy's Sylvester matrix, along both axes."""
    s = O.rht_signs128_from_seed(seed)
    D = np.diag(np.where(_bits(s, d) == 1, -1.0, 1.0))
    T = hadamard(d).astype(np.float64) @ D / np.sqrt(d)
    g = np.random.default_rng(d + seed % 97)
    x = g.standard_normal((2 * d, 3 * d)).astype(np.float32)
    y1 = O.rht(x, 1, d, s).astype(np.float64)
    ref1 = (x.astype(np.float64).reshape(2 * d, 3, d) @ T.T).reshape(2 * d, 3 * d)
    assert np.allclose(y1, ref1, rtol=1e-5, atol=1e-5 * np.abs(x).max())
    y0 = O.rht(x, 0, d, s).astype(np.float64)
    ref0 = np.einsum("ij,bjc->bic", T, x.astype(np.float64).reshape(2, d, 3 * d)).reshape(2 * d, 3 * d)
    assert np.allclose(y0, ref0, rtol=1e-5, atol=1e-5 * np.abs(x).max())


@pytest.mark.parametrize("d", [4, 16, 128])
def test_orthonormal_and_wgrad_identity(d):
    """R^T R = I, so (R dY)^T (R X) = dY^T X along tokens."""
    s = O.rht_signs128_from_seed(3)
    g = np.random.default_rng(1)
    M = 2 * d
    x, dy = g.standard_normal((M, 8)), g.standard_normal((M, 6))
    rx, rdy = O.rht(x, 0, d, s).astype(np.float64), O.rht(dy, 0, d, s).astype(np.float64)
    assert np.allclose(rdy.T @ rx, dy.T @ x, rtol=1e-4, atol=1e-4)
    assert np.allclose(np.linalg.norm(rx, axis=0), np.linalg.norm(x, axis=0), rtol=1e-5)


def test_size16_is_the_recipe_transform():
    """d = 16 with the 128-bit sign block equals the RHT16 of the layer (low
    16 bits of word 0 = rht_signs_from_seed), bit for bit."""
    for seed in (0, 5, 123456789):
        s = O.rht_signs128_from_seed(seed)
        assert int(s[0]) & 0xFFFF == O.rht_signs_from_seed(seed)
        x = np.random.default_rng(seed % 11).standard_normal((32, 48)).astype(np.float32)
        for axis in (0, 1):
            a = O.rht(x, axis, 16, s)
            b = O.rht16(x, axis, O.rht_signs_from_seed(seed))
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_no_randomisation_is_plain_hadamard():
    """Sign option 'none' [Captions Fig. 13]: all-zero sign bits give H_d / sqrt(d)."""
    for d in (4, 16, 128):
        x = np.eye(d, dtype=np.float32)
        y = O.rht(x, 0, d, np.zeros(4, np.uint32)).astype(np.float64)
        assert np.allclose(y, hadamard(d) / np.sqrt(d), atol=1e-7)


def test_seed_per_layer_gives_distinct_signs():
    """Sign option 'a seed per layer': distinct seeds, distinct sign blocks;
    the same seed, the same block."""
    blocks = {tuple(O.rht_signs128_from_seed(s)) for s in range(64)}
    assert len(blocks) == 64
    assert np.array_equal(O.rht_signs128_from_seed(9), O.rht_signs128_from_seed(9))


def test_bad_sizes():
    with pytest.raises(O.OracleError):
        O.rht(np.zeros((8, 8), np.float32), 0, 8, np.zeros(4, np.uint32))
    with pytest.raises(O.OracleError):
        O.rht(np.zeros((100, 128), np.float32), 0, 128, np.zeros(4, np.uint32))
