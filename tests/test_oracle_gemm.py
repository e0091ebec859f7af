"""Pins for the oracle GEMM: exact small-integer special case, a single
16-element block in closed form, entries vs the full matmul, and the
tolerance bound quantity S = sum |a b|."""
import numpy as np

import oracle as O


def _unit_scaled(codes_rows, K):
    """A QTensor whose block scales decode to 1 and g = 1, so deq = E2M1 values."""
    R = codes_rows.shape[0]
    scales = np.full((R, K // 16), 0x38, np.uint8)  # E4M3 0x38 = 1.0
    return O.QTensor(codes_rows, scales, np.float32(1.0), R, K, 0)


def test_gemm_small_integer_exact():
    g = np.random.default_rng(0)
    M, N, K = 8, 6, 64
    a = _unit_scaled(g.integers(0, 256, (M, K // 2), dtype=np.uint8), K)
    b = _unit_scaled(g.integers(0, 256, (N, K // 2), dtype=np.uint8), K)
    C, S = O.gemm(a, b)
    lut = np.array([O.e2m1_decode(c) for c in range(16)])
    def vals(q):
        lo, hi = q.codes & 0xF, q.codes >> 4
        out = np.empty((q.rows, q.cols))
        out[:, 0::2], out[:, 1::2] = lut[lo], lut[hi]
        return out
    A, B = vals(a), vals(b)
    # products of E2M1 values are multiples of 1/4: integer arithmetic is exact
    Ai, Bi = (A * 2).astype(np.int64), (B * 2).astype(np.int64)
    assert np.array_equal(C * 4, (Ai @ Bi.T).astype(np.float64))
    assert np.array_equal(S * 4, (np.abs(Ai) @ np.abs(Bi).T).astype(np.float64))


def test_gemm_single_block_closed_form():
    # K = 16: C = g_a g_b d_a d_b sum_k q_a q_b
    g = np.random.default_rng(1)
    a_codes = g.integers(0, 256, (1, 8), dtype=np.uint8)
    b_codes = g.integers(0, 256, (1, 8), dtype=np.uint8)
    a = O.QTensor(a_codes, np.array([[0x41]], np.uint8), np.float32(0.25), 1, 16, 0)
    b = O.QTensor(b_codes, np.array([[0x2A]], np.uint8), np.float32(3.0), 1, 16, 0)
    lut = [O.e2m1_decode(c) for c in range(16)]
    qa = [lut[(a_codes[0, k // 2] >> (4 * (k % 2))) & 0xF] for k in range(16)]
    qb = [lut[(b_codes[0, k // 2] >> (4 * (k % 2))) & 0xF] for k in range(16)]
    da, db = (1 + 1 / 8) * 2.0 ** (8 - 7), (1 + 2 / 8) * 2.0 ** (5 - 7)
    want = 0.25 * 3.0 * da * db * sum(x * y for x, y in zip(qa, qb))
    C, _ = O.gemm(a, b)
    assert C[0, 0] == want


def test_gemm_entries_match_matmul():
    g = np.random.default_rng(2)
    x = g.standard_normal((32, 96)).astype(np.float32)
    w = (g.standard_normal((48, 96)) * 0.02).astype(np.float32)
    a = O.quantize(x)
    b, _ = O.quantize_2d(w)
    C, S = O.gemm(a, b)
    ms = g.integers(0, 32, 50)
    ns = g.integers(0, 48, 50)
    c, s = O.gemm_entries(O.dequant(a), O.dequant(b), ms, ns)
    assert np.allclose(c, C[ms, ns], rtol=1e-13, atol=1e-13 * S[ms, ns].max())
    assert np.allclose(s, S[ms, ns], rtol=1e-13)
    rows = O.dequant_rows(b, ns)
    assert np.array_equal(rows, O.dequant(b)[ns])


def test_quantised_gemm_close_to_float_gemm():
    """Sanity of the whole chain: the NVFP4 product tracks the unquantised one
    to within FP4's coarse relative error on a typical-magnitude matrix."""
    g = np.random.default_rng(3)
    x = g.standard_normal((64, 256)).astype(np.float32)
    w = g.standard_normal((128, 256)).astype(np.float32)
    C, _ = O.gemm(O.quantize(x), O.quantize_2d(w)[0])
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    rel = np.linalg.norm(C - ref) / np.linalg.norm(ref)
    assert rel < 0.15


def test_tiny_config_oracle_finishes_within_a_second():
    """The tiny configuration end to end on the oracle (A 1x16 RN, B 16x16
    RN, the float64 product, A with stochastic rounding, RHT16 of A along K)
    takes well under a second."""
    import time

    import workloads as W
    a, b = (t.numpy() for t in W.tiny_pair())
    t0 = time.perf_counter()
    qa, (qb, _) = O.quantize(a), O.quantize_2d(b, want_t=False)
    O.gemm(qa, qb)
    O.quantize(a, sr=True, seed=W.SR_SEED, stream=0)
    O.rht16(a, 1, O.rht_signs_from_seed(W.RHT_SEED))
    assert time.perf_counter() - t0 < 1.0
