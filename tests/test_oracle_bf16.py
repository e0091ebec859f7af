"""Pins of the oracle's BF16 forward, the high-precision Fprop of the
precision switch [Review "Core strengths" item 9; Captions Fig. 7].

The oracle computes C = A B^T on the bf16 values in float64.  The pins fix
it against things other than itself: exact rational sums on tiny inputs, a
hand-worked product whose operands are not square (a transposed operand
gives another shape or other numbers), closed forms, the |A||B|^T bound, the
rejection of values bf16 cannot hold, and the recipe composition (the switch
changes only the forward operands)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O


def _bf16_random(rng, shape, spread=8):
    """bf16-representable values over 2^-spread .. 2^spread (truncated fp32)."""
    v = rng.standard_normal(shape) * np.exp2(rng.integers(-spread, spread + 1, shape))
    bits = v.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return bits.view(np.float32)


def test_exact_rational_sums():
    rng = np.random.default_rng(5)
    a = _bf16_random(rng, (5, 7))
    b = _bf16_random(rng, (4, 7))
    C, S = O.bf16_gemm(a, b)
    assert C.shape == (5, 4)
    for m in range(5):
        for n in range(4):
            exact = sum(Fraction(float(a[m, k])) * Fraction(float(b[n, k])) for k in range(7))
            bound = 8 * 2.0 ** -53 * S[m, n]
            assert abs(Fraction(C[m, n]) - exact) <= Fraction(bound)


def test_hand_worked_product():
    a = np.array([[1, 2, 3], [4, 5, 6]], np.float32)
    b = np.array([[1, 0, 0], [0, 1, 0], [0, 0, 1], [1, 1, 1]], np.float32)
    C, S = O.bf16_gemm(a, b)
    assert C.tolist() == [[1, 2, 3, 6], [4, 5, 6, 15]]
    assert S.tolist() == C.tolist()


def test_closed_forms():
    K = 96
    ones = np.ones((3, K), np.float32)
    b = np.repeat(np.arange(1, 6, dtype=np.float32)[:, None], K, axis=1)
    C, _ = O.bf16_gemm(ones, b)
    assert np.array_equal(C, np.tile(K * np.arange(1, 6), (3, 1)))
    # A = the first rows of the identity: C[m, n] = B[n, m]
    rng = np.random.default_rng(6)
    bb = _bf16_random(rng, (6, K))
    eye = np.eye(4, K, dtype=np.float32)
    C, _ = O.bf16_gemm(eye, bb)
    assert np.array_equal(C, bb[:, :4].T.astype(np.float64))


def test_abs_bound_and_signs():
    rng = np.random.default_rng(7)
    a = _bf16_random(rng, (9, 64))
    b = _bf16_random(rng, (11, 64))
    C, S = O.bf16_gemm(a, b)
    assert np.all(S >= np.abs(C))
    C2, S2 = O.bf16_gemm(-a, b)
    assert np.array_equal(C2, -C) and np.array_equal(S2, S)


def test_rejects_values_bf16_cannot_hold():
    assert O.bf16_values(np.float32(1 + 2.0 ** -7)) == 1 + 2.0 ** -7
    with pytest.raises(ValueError):
        O.bf16_values(np.float32(1 + 2.0 ** -10))
    with pytest.raises(O.OracleError):
        O.bf16_gemm(np.ones((2, 32), np.float32), np.ones((2, 48), np.float32))


def test_switch_changes_only_the_forward_operands():
    rng = np.random.default_rng(8)
    M, K, N = 32, 64, 48
    x = _bf16_random(rng, (M, K), 3)
    w = _bf16_random(rng, (N, K), 3) * np.float32(0.02)
    w = (w.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    dy = _bf16_random(rng, (M, N), 3)
    s = O.rht_signs_from_seed(0)
    for two_d in (True, False):
        base = O.linear_operands(x, w, dy, O.Recipe(rht_signs=s, weights_2d=two_d))
        sw = O.linear_operands(x, w, dy, O.Recipe(rht_signs=s, weights_2d=two_d, bf16_fprop=True))
        assert set(base) - set(sw) == {"xq", "wq"}
        for name in sw:
            assert np.array_equal(sw[name].codes, base[name].codes), name
            assert np.array_equal(sw[name].scales, base[name].scales), name
            assert sw[name].g == base[name].g, name
