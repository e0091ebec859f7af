"""Independent, deliberately naive re-statements of the NVFP4 steps, used only
to pin the oracle on tiny inputs.  Nothing here calls the oracle's arithmetic:
tables come from the golden fixtures or from the format definitions, rounding
is an argmin over the value table, and stochastic-rounding thresholds are
exact rationals.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def e2m1_table():
    vals = []
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.append(Fraction(line))
    assert len(vals) == 8
    return vals


def e4m3_table():
    """All non-negative finite OCP E4M3FN values, index = code (0..126).
    Built by enumerating sign-free bit patterns: exponent field e (bias 7),
    mantissa field f; e == 0 is subnormal (f/8 * 2^-6); code 127 is NaN."""
    out = []
    for code in range(127):
        e, f = code >> 3, code & 7
        if e == 0:
            out.append(Fraction(f, 8) * Fraction(1, 64))
        else:
            out.append((1 + Fraction(f, 8)) * (Fraction(2) ** (e - 7)))
    return out


E2M1 = e2m1_table()
E4M3 = e4m3_table()


def nearest_even(value: Fraction, table) -> int:
    """Index of the nearest table entry; ties go to the even index; beyond
    the largest entry saturate to it."""
    best, best_d = None, None
    for i, t in enumerate(table):
        d = abs(value - t)
        if best is None or d < best_d or (d == best_d and i % 2 == 0 and best % 2 == 1):
            best, best_d = i, d
    return best


def sr_index(m: Fraction, r16: int) -> int:
    """Round up iff 64 * r16 < floor(frac * 2^22) (fraction in 22-bit fixed point)."""
    if m >= E2M1[-1]:
        return 7
    lo = max(i for i, t in enumerate(E2M1) if t <= m)
    frac = (m - E2M1[lo]) / (E2M1[lo + 1] - E2M1[lo])
    T = (frac * 2**22).numerator // (frac * 2**22).denominator
    return lo + 1 if 64 * r16 < T else lo


# ---------------------------------------------------------------- Philox4x32-10
M0, M1, W0, W1 = 0xD2511F53, 0xCD9E8D57, 0x9E3779B9, 0xBB67AE85
MASK = 0xFFFFFFFF


def philox(ctr, key, rounds=10):
    c = list(ctr)
    k0, k1 = key
    for _ in range(rounds):
        p0 = M0 * c[0]
        p1 = M1 * c[2]
        c = [((p1 >> 32) ^ c[1] ^ k0) & MASK, p1 & MASK, ((p0 >> 32) ^ c[3] ^ k1) & MASK, p0 & MASK]
        k0 = (k0 + W0) & MASK
        k1 = (k1 + W1) & MASK
    return c


def sr_bits(seed, stream, e):
    j = e // 8
    out = philox([j & MASK, j >> 32, stream, 0], [seed & MASK, seed >> 32])
    h = e % 8
    w = out[h // 2]
    return (w & 0xFFFF) if h % 2 == 0 else (w >> 16)


# ---------------------------------------------------------------- quantise
def hadamard16():
    H = np.ones((1, 1))
    while H.shape[0] < 16:
        H = np.block([[H, H], [H, -H]])
    return H


def f32(v):
    return np.float32(v)


def quantize_block(vals, s_enc, s6, rbits=None):
    """vals: list of np.float32.  Returns (scale code, list of 4-bit codes)."""
    amax_b = max(abs(v) for v in vals)
    t = f32(amax_b * s6)
    d_code = nearest_even(Fraction(float(t)), E4M3) if t < f32(448.0) else 126
    d = f32(float(E4M3[d_code]))
    r = f32(0.0) if d == 0 else f32(s_enc / d)
    codes = []
    for i, x in enumerate(vals):
        v = f32(x * r)
        m = Fraction(float(abs(v)))
        idx = nearest_even(m, E2M1) if rbits is None else sr_index(m, rbits[i])
        sign = 8 if np.signbit(x) else 0
        codes.append(sign | idx)
    return d_code, codes


def tensor_scales(op):
    amax = f32(np.max(np.abs(op)))
    if amax == 0:
        return f32(1.0), f32(1.0) / f32(6.0), f32(1.0)
    s_enc = f32(f32(2688.0) / amax)
    return s_enc, f32(s_enc / f32(6.0)), f32(f32(1.0) / s_enc)


def quantize(x, transpose=False, rht=False, signs=0, sr=False, seed=0, offset=0, stream=0):
    """Slow restatement of 1x16 quantisation.  With rht, inputs must make the
    transform exact in fp32 (the matrix form is evaluated in float64)."""
    op = np.array(x, dtype=np.float32)
    if transpose:
        op = op.T.copy()
    R, C = op.shape
    if rht:
        D = np.diag([-1.0 if (signs >> i) & 1 else 1.0 for i in range(16)])
        T = 0.25 * hadamard16() @ D
        op64 = op.astype(np.float64).reshape(R, C // 16, 16) @ T.T
        op = op64.reshape(R, C).astype(np.float32)
        assert np.array_equal(op.astype(np.float64), op64.reshape(R, C)), "RHT not exact"
    s_enc, s6, g = tensor_scales(op)
    codes = np.zeros((R, C // 2), np.uint8)
    scales = np.zeros((R, C // 16), np.uint8)
    for i in range(R):
        for b in range(C // 16):
            vals = [op[i, b * 16 + t] for t in range(16)]
            rb = None
            if sr:
                rb = [sr_bits(seed, stream, offset + i * C + b * 16 + t) for t in range(16)]
            d, cs = quantize_block(vals, s_enc, s6, rb)
            scales[i, b] = d
            for t in range(8):
                codes[i, b * 8 + t] = cs[2 * t] | (cs[2 * t + 1] << 4)
    return codes, scales, g


def quantize_2d(w):
    w = np.array(w, dtype=np.float32)
    R, C = w.shape
    s_enc, s6, g = tensor_scales(w)
    full = np.zeros((R, C), np.uint8)
    grid = np.zeros((R // 16, C // 16), np.uint8)
    for bi in range(R // 16):
        for bj in range(C // 16):
            vals = [w[bi * 16 + r, bj * 16 + c] for r in range(16) for c in range(16)]
            d, cs = quantize_block(vals, s_enc, s6)
            grid[bi, bj] = d
            full[bi * 16:bi * 16 + 16, bj * 16:bj * 16 + 16] = np.array(cs, np.uint8).reshape(16, 16)
    codes = full[:, 0::2] | (full[:, 1::2] << 4)
    return codes, grid, g


def decode(codes, scales, g, mode=0):
    R, C2 = codes.shape
    C = 2 * C2
    out = np.zeros((R, C))
    for i in range(R):
        for j in range(C):
            byte = int(codes[i, j // 2])
            c = byte & 0xF if j % 2 == 0 else byte >> 4
            mag = float(E2M1[c & 7])
            sc = scales[i, j // 16] if mode == 0 else scales[i // 16, j // 16]
            out[i, j] = (-mag if c & 8 else mag) * float(E4M3[int(sc)]) * float(g)
    return out
