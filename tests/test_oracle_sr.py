"""Pins for stochastic rounding and its counter-based random source:
the page's SR mini-example, exact enumeration of the probability, the
unbiasedness statistic, Philox known-answer vectors and uniformity."""
import os

import numpy as np
import pytest

import oracle as O
from tests import bruteforce as BF
from tests.test_oracle_quantize import _toy

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                v = [int(t, 16) for t in line.split()]
                rows.append((v[0:4], v[4:6], v[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,want", _kat())
def test_philox_known_answers(ctr, key, want):
    assert list(O.philox4x32_10(ctr, key)) == want
    assert BF.philox(ctr, key) == want


def test_sr_bits_layout():
    # element e takes 16-bit half (e mod 8) of the call with counter e // 8
    seed, stream = 0x123456789ABCDEF0, 5
    for e in [0, 1, 7, 8, 15, 2**33 + 3]:
        j = e // 8
        out = O.philox4x32_10([j & 0xFFFFFFFF, j >> 32, stream, 0],
                              [seed & 0xFFFFFFFF, seed >> 32])
        w = out[(e % 8) // 2]
        want = (w & 0xFFFF) if e % 2 == 0 else (w >> 16)
        assert O.sr_bits(seed, stream, e) == want == BF.sr_bits(seed, stream, e)


def _count_up(m):
    r = np.arange(65536, dtype=np.uint32)
    idx = O.e2m1_sr_index_n(np.full(65536, m, np.float32), r)
    return idx


@pytest.mark.parametrize("m", [0.1, 0.26, 0.5, 0.74, 1.03, 1.2499, 1.6, 2.2, 2.9999, 3.5, 4.7, 5.99,
                               3e-4, 1.7e-6, 2.0 ** -30])
def test_sr_exact_enumeration(m):
    """Over all 2^16 values of the 16-bit draw the round-up count equals
    ceil(T / 64) with T = floor(frac * 2^22), frac = (m - lo)/(hi - lo)
    computed exactly: probability T / 2^22 to within one 2^-16 step."""
    from fractions import Fraction
    m32 = np.float32(m)
    idx = _count_up(m32)
    tv = BF.E2M1
    mf = Fraction(float(m32))
    lo = max(i for i, t in enumerate(tv) if t <= mf)
    frac = (mf - tv[lo]) / (tv[lo + 1] - tv[lo])
    T = int(frac * 2**22)  # floor (frac >= 0)
    n_up = int((idx == lo + 1).sum())
    assert set(np.unique(idx)) <= {lo, lo + 1}
    assert n_up == -(-T // 64)
    assert abs(n_up / 65536 - float(frac)) <= 2.0 ** -16


def test_sr_22bit_fraction_boundaries():
    """The fraction is kept to 22 bits: for |v| >= 1 that is every mantissa
    bit below the E2M1 bit (no truncation); below 1 the lower bits drop."""
    # 1 + 64*k * 2^-23 has T = 64k: draw r16 = k is the first not rounding up
    for k in (1, 7, 1000):
        m = np.float32(1.0 + 64 * k * 2.0 ** -22 / 2)
        assert O.e2m1_sr_index(m, k - 1) == 3 and O.e2m1_sr_index(m, k) == 2
    # a magnitude whose fraction has bits only below 2^-22 never rounds up
    assert O.e2m1_sr_index(np.float32(2.0 ** -30), 0) == 0
    # just above a multiple of 64 / 2^22 in the subnormal range: truncated to it
    m = np.float32((64 * 3 + 0.5) * 2.0 ** -23)   # frac * 2^22 = 192.5 -> T = 192
    assert O.e2m1_sr_index(m, 2) == 1 and O.e2m1_sr_index(m, 3) == 0


def test_sr_page_mini_example():
    """Page SR mini-example: 1.03 between 1 and 1.5 rounds to 1 with
    probability 0.94 and to 1.5 with 0.06 (to the page's two digits), and the
    expectation is 1.03."""
    v, lo, hi, p_lo, p_hi = _toy()["sr"][0]
    idx = _count_up(np.float32(v))
    vals = np.array([O.e2m1_decode(int(i)) for i in idx])
    assert set(np.unique(vals)) == {lo, hi}
    f_hi = np.mean(vals == hi)
    assert abs(f_hi - p_hi) < 0.005 and abs((1 - f_hi) - p_lo) < 0.005
    assert abs(vals.mean() - v) < 2 ** -16


def test_sr_saturation_and_grid_points():
    for m in (6.0, 6.5, 1e9):
        assert set(np.unique(_count_up(np.float32(m)))) == {7}
    for i, t in enumerate([0, .5, 1, 1.5, 2, 3, 4]):
        assert set(np.unique(_count_up(np.float32(t)))) == {i}  # exact grid values never move


def test_sr_unbiased_over_seeded_draws():
    """1e5 seeded draws per value through the counter-based stream: the mean
    of the rounded values is within 5 sigma of the input."""
    n = 100_000
    for k, v in enumerate([0.13, 0.61, 1.03, 1.37, 2.71, 3.3, 4.9, 5.5]):
        r = O.sr_bits_n(1234, 0, k * n, n)
        idx = O.e2m1_sr_index_n(np.full(n, v, np.float32), r)
        vals = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])[idx]
        lo, hi = vals.min(), vals.max()
        p = (v - lo) / (hi - lo) if hi > lo else 0.0
        sigma = (hi - lo) * np.sqrt(p * (1 - p) / n) + 1e-12
        assert abs(vals.mean() - v) < 5 * sigma, (v, vals.mean(), sigma)


def test_sr_stream_is_uniform():
    """Chi-square of 16-bit halves in 256 bins and of their low bytes."""
    r = O.sr_bits_n(42, 0, 0, 1 << 20)
    for vals, bins in ((r >> 8, 256), (r & 0xFF, 256)):
        h = np.bincount(vals.astype(np.int64), minlength=bins)
        exp = r.size / bins
        chi2 = ((h - exp) ** 2 / exp).sum()
        assert chi2 < bins - 1 + 6 * np.sqrt(2 * (bins - 1))
    # different streams and seeds give different draws
    assert not np.array_equal(O.sr_bits_n(42, 1, 0, 64), r[:64])
    assert not np.array_equal(O.sr_bits_n(43, 0, 0, 64), r[:64])


def test_rht_signs_from_seed():
    assert O.rht_signs_from_seed(0) == O.philox4x32_10([0, 0, 0, 0], [0, 0])[0] & 0xFFFF
    assert O.rht_signs_from_seed(0) == 0xE8D5  # low half of the first KAT word


def test_sr_probability_dense_grid():
    """[Review s10 SR formula; s4]: P(round up) = (|v| - lo) / (hi - lo).
    Over a dense grid of magnitudes in every E2M1 interval -- [0, 0.5) down
    to 2^-40, [0.5, 1) and [1, 1.5) where the 22-bit fraction and the fp32
    spacing interact, up to [4, 6) -- and the fp32 neighbours of every grid
    point, the round-up share over all 2^16 draws lies within 2^-16 of that
    exact probability; at and above 6 the code is always 6."""
    from fractions import Fraction
    rng = np.random.default_rng(20250)
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    vals = []
    for lo, hi in zip(grid[:-1], grid[1:]):
        vals += list(rng.uniform(lo, hi, 48).astype(np.float32))
        for p in (lo, hi):
            f = np.float32(p)
            vals += [np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(7))]
    vals += list(np.float32(2.0) ** rng.uniform(-40, -1, 48).astype(np.float32))
    vals = np.unique(np.array([v for v in vals if 0 < v < 6], np.float32))
    r = np.tile(np.arange(65536, dtype=np.uint32), 1)
    worst = 0.0
    for i in range(0, vals.size, 32):
        chunk = vals[i:i + 32]
        m = np.repeat(chunk, 65536)
        idx = O.e2m1_sr_index_n(m, np.tile(r, chunk.size)).reshape(chunk.size, 65536)
        for v, row in zip(chunk, idx):
            vf = Fraction(float(v))
            lo = max(k for k, t in enumerate(grid) if Fraction(t) <= vf)
            frac = (vf - Fraction(grid[lo])) / (Fraction(grid[lo + 1]) - Fraction(grid[lo]))
            assert set(np.unique(row)) <= {lo, lo + 1}, v
            p_up = Fraction(int((row == lo + 1).sum()), 65536)
            worst = max(worst, abs(float(p_up - frac)))
            assert abs(p_up - frac) <= Fraction(1, 65536), (float(v), float(p_up), float(frac))
    assert worst > 0  # the grid does reach the 16-bit resolution limit somewhere
    for v in (6.0, 6.5, 100.0, 3e38):
        idx = O.e2m1_sr_index_n(np.full(4096, v, np.float32), np.arange(4096, dtype=np.uint32) * 16)
        assert np.all(idx == 7)
