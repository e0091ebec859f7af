"""Pins of the oracle's MXFP4 comparator (CPU only).

MXFP4 as the pages describe it [Review "secret weapon" items 1-2; Captions
Fig. 6]: blocks of 32 E2M1 values with one power-of-two (UE8M0) scale, no tensor scale; the
pages attribute MXFP4's extra loss to that power-of-two rounding losing a
binade around +-4 / +-6.  The scale rule is the OCP Microscaling one,
e = floor(log2(amax)) - 2 (a reading; the pages do not spell it out), and the
tests below pin the oracle against an independent restatement in exact
rational arithmetic, closed forms and invariants.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def ref_block(xs):
    """Independent restatement: exact rationals, frexp for the exponent,
    nearest grid value with ties to the even index, saturation at 6."""
    xs = [float(np.float32(v)) for v in xs]
    amax = max(abs(v) for v in xs)
    if amax == 0:
        e = -127
    else:
        m, ex = math.frexp(amax)  # amax = m 2^ex, m in [0.5, 1)
        e = max(-127, min(127, (ex - 1) - 2))
    codes = []
    for v in xs:
        q = abs(Fraction(v)) / (Fraction(2) ** e)
        if q >= 6:
            idx = 7
        else:
            best = min(range(8), key=lambda i: (abs(GRID[i] - q), i % 2))
            idx = best
        codes.append((8 if math.copysign(1.0, v) < 0 else 0) | idx)
    return e + 127, codes


def test_binade_loss_example():
    """The page's lost binade: a block whose amax lies in [6, 8) x 2^k keeps a
    scale of 2^k, so its largest values saturate to 6 x 2^k."""
    for k in (-3, 0, 5):
        s = 2.0 ** k
        sc, codes = O.mx_block([7.0 * s, 6.5 * s, 5.0 * s, 3.5 * s])
        assert sc == 127 + k
        assert list(codes[:4]) == [7, 7, 6, 6]  # 7->6, 6.5->6, 5 tie->4, 3.5 tie->4
        # NVFP4 maps the same block's amax exactly onto the FP4 maximum
        q = O.quantize(np.array([[7.0 * s, 6.5 * s, 5.0 * s, 3.5 * s] + [0.0] * 12], np.float32))
        assert q.codes[0, 0] & 0xF == 7 and np.isclose(O.dequant(q)[0, 0], 7.0 * s, rtol=0.07)


@pytest.mark.parametrize("amax", [1.0, 1.5, 3.999, 4.0, 6.0, 7.99, 8.0, 1e-30, 3e38, 2.0 ** -126,
                                  2.0 ** -140])
def test_scale_closed_form(amax):
    sc, _ = O.mx_block([np.float32(amax), 0.0])
    a = float(np.float32(amax))
    e = math.frexp(a)[1] - 1 - 2
    assert sc == max(0, min(254, e + 127))
    # every element's scaled magnitude lies below 8 and the amax lands in [4, 8)
    if e > -127:
        assert 4.0 <= a / 2.0 ** e < 8.0


def test_brute_force_blocks():
    g = np.random.default_rng(3)
    for trial in range(300):
        n = 32
        x = (g.standard_normal(n) * 10.0 ** g.uniform(-6, 6)).astype(np.float32)
        if trial % 5 == 0:  # exact ties and grid points
            x = (g.integers(-16, 17, n) * 0.25 * 2.0 ** g.integers(-8, 8)).astype(np.float32)
        sc, codes = O.mx_block(x)
        rsc, rcodes = ref_block(x)
        assert sc == rsc, trial
        assert list(codes) == rcodes, trial


def test_power_of_two_invariance():
    g = np.random.default_rng(4)
    x = g.standard_normal((8, 64)).astype(np.float32)
    q0 = O.mx_quantize(x)
    for j in (-7, 3, 20):
        q = O.mx_quantize(x * np.float32(2.0 ** j))
        assert np.array_equal(q.codes, q0.codes)
        assert np.array_equal(q.scales.astype(int), q0.scales.astype(int) + j)


def test_zero_and_nonfinite_blocks():
    sc, codes = O.mx_block(np.zeros(32, np.float32))
    assert sc == 0 and not codes.any()
    x = np.ones(32, np.float32)
    x[5] = np.nan
    assert O.mx_block(x)[0] == 0xFF
    assert math.isnan(O.e8m0_decode(0xFF)) and O.e8m0_decode(127) == 1.0


def test_quantize_layout_and_dequant():
    g = np.random.default_rng(5)
    x = g.standard_normal((3, 96)).astype(np.float32)
    q = O.mx_quantize(x)
    deq = O.mx_dequant(q)
    for r in range(3):
        for b in range(3):
            sc, codes = ref_block(x[r, 32 * b:32 * b + 32])
            assert q.scales[r, b] == sc
            for j in range(32):
                byte = q.codes[r, 16 * b + j // 2]
                assert (byte >> (4 * (j % 2))) & 0xF == codes[j]
                v = float(GRID[codes[j] & 7]) * (-1 if codes[j] & 8 else 1) * 2.0 ** (sc - 127)
                assert deq[r, 32 * b + j] == v
    # reconstruction: |x - x_hat| <= half the grid spacing at |x| / X (0.5 below
    # 2, 1 below 4, 2 below 6), or |x| >= 6 X and x_hat = +-6 X
    X = np.repeat(2.0 ** (q.scales.astype(np.float64) - 127), 32, axis=1)
    m = np.abs(x) / X
    half = np.where(m < 2, 0.25, np.where(m < 4, 0.5, 1.0)) * X
    sat = (m >= 6) & (np.abs(deq) == 6 * X)
    assert np.all((np.abs(deq - x) <= half) | sat)


def test_gemm_matches_exact_sum():
    g = np.random.default_rng(6)
    a, b = g.standard_normal((4, 64)), g.standard_normal((5, 64))
    qa, qb = O.mx_quantize(a), O.mx_quantize(b)
    C, S = O.mx_gemm(qa, qb)
    ah, bh = O.mx_dequant(qa), O.mx_dequant(qb)
    for m in range(4):
        for n in range(5):
            exact = sum(Fraction(float(ah[m, k])) * Fraction(float(bh[n, k])) for k in range(64))
            assert C[m, n] == pytest.approx(float(exact), rel=1e-15, abs=1e-300)
            assert S[m, n] >= abs(C[m, n])
