"""Targeted pins for the fp32 operation order of the scale steps and for
exact rounding ties.  The order is a stated reading (t = amax_b * (s_enc/6),
r_b = s_enc / d_b, v = x * r_b, each one rounded fp32 operation); these tests
search for inputs where the mathematically equal alternatives round
differently and check the oracle follows the stated order exactly."""
import numpy as np

import oracle as O
from tests import bruteforce as BF
from tests.test_oracle_formats import _bisect_nearest_even

f32 = np.float32


def _e4m3(t):
    t = np.asarray(t, np.float32)
    out = _bisect_nearest_even(t, BF.E4M3)
    return np.where(t >= f32(448.0), 126, out)


def test_unit_multiplier_block_ties():
    """A tensor with amax 6 has s_enc = 448 and its amax block gets d_b = 448,
    so that block's multiplier is exactly 1 and v = x: the E2M1 midpoints then
    exercise nearest-even ties directly."""
    x = np.zeros((1, 16), np.float32)
    vals = [6.0, 2.5, -0.25, 1.25, 1.75, 3.5, -5.0, 0.75, 4.5, 0.3]
    x[0, :len(vals)] = vals
    q = O.quantize(x)
    assert q.scales[0, 0] == 0x7E and q.g == f32(1.0) / f32(448.0)
    want = [6.0, 2.0, -0.0, 1.0, 2.0, 4.0, -4.0, 1.0, 4.0, 0.5]
    for j, w in enumerate(want):
        c = (q.codes[0, j // 2] >> (4 * (j % 2))) & 0xF
        got = O.e2m1_decode(int(c))
        assert got == w and np.signbit(got) == np.signbit(w), (vals[j], got, w)


def _search_scale_order_cases(n=4000, seed=0):
    """Candidates placed within a few fp32 ulps of an E4M3 midpoint, so that a
    one-ulp difference in t decides the block scale."""
    g = np.random.default_rng(seed)
    tv = np.array([float(v) for v in BF.E4M3])
    mids = ((tv[1:] + tv[:-1]) / 2)[8:]          # normal-range midpoints
    A = (f32(2.0) ** g.uniform(-20, 20, n)).astype(np.float32)
    s_enc = (f32(2688.0) / A).astype(np.float32)
    s6 = (s_enc / f32(6.0)).astype(np.float32)
    mid = mids[g.integers(0, mids.size, n)]
    base = (mid / s6).astype(np.float32)
    out_a, out_b, out_c = [], [], []
    for k in range(-6, 7):
        ab = (base * (f32(1.0) + f32(k) * f32(2.0 ** -23))).astype(np.float32)
        ok = ab <= A
        t_ref = (ab * s6).astype(np.float32)
        t_alt1 = (ab * (f32(448.0) / A).astype(np.float32)).astype(np.float32)
        t_alt2 = ((ab * s_enc).astype(np.float32) / f32(6.0)).astype(np.float32)
        c_ref, c1, c2 = _e4m3(t_ref), _e4m3(t_alt1), _e4m3(t_alt2)
        hit = np.nonzero(ok & ((c_ref != c1) | (c_ref != c2)))[0]
        out_a.append(A[hit]); out_b.append(ab[hit]); out_c.append(c_ref[hit])
    return np.concatenate(out_a), np.concatenate(out_b), np.concatenate(out_c)


def test_block_scale_operation_order():
    A, ab, c_ref = _search_scale_order_cases()
    assert A.size >= 3, "search found too few discriminating cases"
    for a, b, c in list(zip(A, ab, c_ref))[:40]:
        x = np.zeros((1, 32), np.float32)
        x[0, 0] = a
        x[0, 16] = b
        q = O.quantize(x)
        assert q.scales[0, 1] == c, (a, b)


def test_element_multiplier_operation_order():
    """v = x * (s_enc / d_b) rounded per step; search x where the alternative
    (x * s_enc) / d_b lands on the other side of an E2M1 decision point."""
    g = np.random.default_rng(1)
    found = 0
    for trial in range(400):
        A = f32(2.0 ** g.uniform(-8, 8))
        s_enc = f32(f32(2688.0) / A)
        s6 = f32(s_enc / f32(6.0))
        ab = f32(A * f32(g.uniform(0.05, 1.0)))
        d_code = int(_e4m3([f32(ab * s6)])[0])
        d = f32(float(BF.E4M3[d_code]))
        if d == 0:
            continue
        r = f32(s_enc / d)
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
        # candidates x near each decision point / r
        cand = (mids[:, None] / r * (1 + np.arange(-64, 65, dtype=np.float32) * f32(2 ** -23))).astype(np.float32).ravel()
        cand = cand[np.abs(cand) <= ab]
        v_ref = (cand * r).astype(np.float32)
        v_alt = ((cand * s_enc).astype(np.float32) / d).astype(np.float32)
        i_ref = _bisect_nearest_even(np.abs(v_ref), BF.E2M1)
        i_alt = _bisect_nearest_even(np.abs(v_alt), BF.E2M1)
        sel = np.nonzero(i_ref != i_alt)[0][:4]
        for k in sel:
            x = np.zeros((1, 32), np.float32)
            x[0, 0] = A
            x[0, 16] = ab
            x[0, 17] = cand[k]
            q = O.quantize(x)
            assert q.scales[0, 1] == d_code
            c = q.codes[0, 8] >> 4
            assert c & 7 == i_ref[k], (A, ab, cand[k])
            found += 1
        if found >= 20:
            break
    assert found >= 5
