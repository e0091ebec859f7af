"""Pins for the oracle's number formats: E2M1 decode/encode and E4M3
encode/decode, checked against the page's printed value set and against
brute-force argmin over independently built value tables."""
import numpy as np
import pytest

import oracle as O
from tests import bruteforce as BF


def test_e2m1_decode_matches_printed_value_set():
    # Page value set (golden fixture): +-{0, .5, 1, 1.5, 2, 3, 4, 6}
    for c in range(16):
        mag = float(BF.E2M1[c & 7])
        want = -mag if c & 8 else mag
        got = O.e2m1_decode(c)
        assert got == want and np.signbit(got) == bool(c & 8)


def test_e4m3_table_closed_form_facts():
    # OCP E4M3FN facts: 0x7E is 448 (largest finite), 0x08 is 2^-6 (smallest
    # normal), 0x01 is 2^-9 (smallest subnormal), 0x38 is 1.0, values strictly
    # increase with the code, 0x7F is NaN.
    assert O.e4m3_decode(0x7E) == 448.0
    assert O.e4m3_decode(0x08) == 2.0 ** -6
    assert O.e4m3_decode(0x01) == 2.0 ** -9
    assert O.e4m3_decode(0x38) == 1.0
    assert np.isnan(O.e4m3_decode(0x7F))
    vals = [O.e4m3_decode(c) for c in range(127)]
    assert all(b > a for a, b in zip(vals, vals[1:]))
    assert [float(v) for v in BF.E4M3] == vals
    assert O.e4m3_decode(0x80 | 0x38) == -1.0


def _critical_points(table):
    """Every table value and every midpoint, with their fp32 neighbours."""
    pts = []
    tv = [float(v) for v in table]
    for a, b in zip(tv, tv[1:]):
        for c in (a, (a + b) / 2):
            c32 = np.float32(c)
            pts += [np.nextafter(c32, np.float32(-1)), c32, np.nextafter(c32, np.float32(np.inf))]
    pts.append(np.float32(tv[-1]))
    pts += [np.float32(tv[-1] * 1.03), np.float32(tv[-1] * 7.0), np.float32(3e38)]
    return np.array([p for p in pts if p >= 0], np.float32)


def _bisect_nearest_even(vals, table):
    tv = np.array([float(v) for v in table])
    v64 = vals.astype(np.float64)
    hi = np.searchsorted(tv, v64, side="left").clip(1, len(tv) - 1)
    lo = hi - 1
    dlo, dhi = v64 - tv[lo], tv[hi] - v64
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(v64 >= tv[-1], len(tv) - 1, pick)
    pick = np.where(v64 <= tv[0], 0, pick)
    return pick.astype(np.uint8)


def _stride_sample(lo_bits, hi_bits, stride):
    bits = np.arange(lo_bits, hi_bits, stride, dtype=np.uint64).astype(np.uint32)
    return bits.view(np.float32)


def test_e4m3_encode_brute_force():
    # Decision boundaries exhaustively, plus every 127th fp32 bit pattern from 0
    # up to +inf: compared with an argmin over the 127-entry table
    # (ties to the even code, saturation at 448).
    crit = _critical_points(BF.E4M3)
    sample = _stride_sample(0, 0x7F800000, 127)
    vals = np.concatenate([crit, sample])
    got = O.e4m3_encode_n(vals)
    want = _bisect_nearest_even(vals, BF.E4M3)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (vals[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e4m3_encode_ties_and_saturation():
    assert O.e4m3_encode(2.0 ** -10) == 0          # tie 0 / 2^-9 -> even code 0
    assert O.e4m3_encode(3 * 2.0 ** -10) == 2      # tie 2^-9 / 2^-8 -> code 2
    assert O.e4m3_encode(1.0 + 1.0 / 16) == 0x38   # tie 1 / 1.125 -> code 0x38
    assert O.e4m3_encode(1.0 + 3.0 / 16) == 0x3A   # tie 1.125 / 1.25 -> 0x3A
    assert O.e4m3_encode(447.99997) == 0x7E
    assert O.e4m3_encode(460.0) == 0x7E
    assert O.e4m3_encode(1e30) == 0x7E
    assert O.e4m3_encode(0.0) == 0


def test_e2m1_rn_brute_force():
    crit = _critical_points(BF.E2M1)
    sample = _stride_sample(0, 0x41400000, 37)  # 0 .. 12
    vals = np.concatenate([crit, sample])
    got = O.e2m1_rn_index_n(vals)
    want = _bisect_nearest_even(vals, BF.E2M1)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (vals[bad[:5]], got[bad[:5]], want[bad[:5]])


@pytest.mark.parametrize("m,idx", [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4),
                                   (3.5, 6), (5.0, 6), (6.0, 7), (100.0, 7), (0.0, 0)])
def test_e2m1_rn_ties(m, idx):
    # Exact midpoints go to the even code (the page's nearest-even rule).
    assert O.e2m1_rn_index(m) == idx


def test_e2m1_rn_monotone():
    vals = np.sort(np.concatenate([_stride_sample(0, 0x41000000, 101),
                                   _critical_points(BF.E2M1)]))
    idx = O.e2m1_rn_index_n(vals)
    assert np.all(np.diff(idx.astype(int)) >= 0)
