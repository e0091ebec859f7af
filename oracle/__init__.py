"""NVFP4 CPU oracle -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-checkable CPU statement of the NVFP4 linear layer:
two-level quantisation (FP32 tensor scale, E4M3 1x16 or 16x16 block scale,
E2M1 codes, nearest-even or stochastic rounding), the 16-point random
Hadamard transform, dequantisation and float64 GEMMs of dequantised operands.
The arithmetic lives in ``nvfp4_oracle.c`` (fp32 steps exactly as the pages
order them); this module only marshals numpy arrays and composes the layer.

Only the test-suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package.  It shares no code with the GPU library
and does not import it.

Citations: [Review] is the web page "NVFP4 4-bit Pretraining, Made Practical:
12B up to 10T Tokens, Effectively On Par with FP8" (a review of Pretraining
Large Language Models with NVFP4, arXiv 2509.25149), cited by its numbered
sections; [Captions] is that paper's figure-caption list.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = ctypes.CDLL(path)
        u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
        f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
        f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
        u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
        i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
        i64, u64, u32, i32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int
        L.oracle_e2m1_decode.restype = ctypes.c_double
        L.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e2m1_rn_index.restype = i32
        L.oracle_e2m1_rn_index.argtypes = [ctypes.c_float]
        L.oracle_e2m1_sr_index.restype = i32
        L.oracle_e2m1_sr_index.argtypes = [ctypes.c_float, u32]
        L.oracle_philox4x32_10.restype = None
        L.oracle_philox4x32_10.argtypes = [u32p, u32p, u32p]
        L.oracle_sr_bits.restype = u32
        L.oracle_sr_bits.argtypes = [u64, u32, u64]
        L.oracle_rht_signs_from_seed.restype = u32
        L.oracle_rht_signs_from_seed.argtypes = [u64]
        L.oracle_rht16_chunk.restype = None
        L.oracle_rht16_chunk.argtypes = [f32p, u32, f32p]
        L.oracle_rht16.restype = i32
        L.oracle_rht16.argtypes = [f32p, i64, i64, i64, i32, u32, f32p]
        L.oracle_quantize.restype = i32
        L.oracle_quantize.argtypes = [f32p, i64, i64, i64, i32, i32, u32, i32, u64, u64,
                                      u32, u8p, u8p, ctypes.POINTER(ctypes.c_float)]
        L.oracle_quantize_2d.restype = i32
        L.oracle_quantize_2d.argtypes = [f32p, i64, i64, i64, u8p, u8p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
        L.oracle_dequant.restype = None
        L.oracle_dequant.argtypes = [u8p, u8p, ctypes.c_float, i64, i64, i32, f64p]
        L.oracle_gemm_entries.restype = None
        L.oracle_gemm_entries.argtypes = [f64p, f64p, i64, i64p, i64p, i64, f64p, f64p]
        L.oracle_e4m3_encode_n.restype = None
        L.oracle_e4m3_encode_n.argtypes = [f32p, i64, u8p]
        L.oracle_e2m1_rn_index_n.restype = None
        L.oracle_e2m1_rn_index_n.argtypes = [f32p, i64, u8p]
        L.oracle_e2m1_sr_index_n.restype = None
        L.oracle_e2m1_sr_index_n.argtypes = [f32p, u32p, i64, u8p]
        L.oracle_sr_bits_n.restype = None
        L.oracle_sr_bits_n.argtypes = [u64, u32, u64, i64, u32p]
        L.oracle_rht_signs128_from_seed.restype = None
        L.oracle_rht_signs128_from_seed.argtypes = [u64, u32p]
        L.oracle_rht_d.restype = i32
        L.oracle_rht_d.argtypes = [f32p, i64, i64, i64, i32, i32, u32p, f32p]
        L.oracle_mx_block.restype = ctypes.c_uint8
        L.oracle_mx_block.argtypes = [f32p, i32, u8p]
        L.oracle_mx_quantize.restype = i32
        L.oracle_mx_quantize.argtypes = [f32p, i64, i64, i64, u8p, u8p]
        L.oracle_e8m0_decode.restype = ctypes.c_double
        L.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
        L.oracle_mx_dequant.restype = None
        L.oracle_mx_dequant.argtypes = [u8p, u8p, i64, i64, f64p]
        _lib = L
    return _lib


class OracleError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"oracle status {status}")
        self.status = status


ERR_SHAPE = 2
ERR_NONFINITE = 7

# ---------------------------------------------------------------- scalars


def e2m1_decode(code: int) -> float:
    return lib().oracle_e2m1_decode(code)


def e4m3_decode(b: int) -> float:
    return lib().oracle_e4m3_decode(b)


def e4m3_encode(t: float) -> int:
    return int(lib().oracle_e4m3_encode(t))


def e2m1_rn_index(m: float) -> int:
    return int(lib().oracle_e2m1_rn_index(m))


def e2m1_sr_index(m: float, r16: int) -> int:
    return int(lib().oracle_e2m1_sr_index(m, r16))


def e4m3_encode_n(t: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.float32).ravel()
    out = np.empty(t.size, np.uint8)
    lib().oracle_e4m3_encode_n(t, t.size, out)
    return out


def e2m1_rn_index_n(m: np.ndarray) -> np.ndarray:
    m = np.ascontiguousarray(m, dtype=np.float32).ravel()
    out = np.empty(m.size, np.uint8)
    lib().oracle_e2m1_rn_index_n(m, m.size, out)
    return out


def e2m1_sr_index_n(m: np.ndarray, r16: np.ndarray) -> np.ndarray:
    m = np.ascontiguousarray(m, dtype=np.float32).ravel()
    r = np.ascontiguousarray(r16, dtype=np.uint32).ravel()
    assert r.size == m.size
    out = np.empty(m.size, np.uint8)
    lib().oracle_e2m1_sr_index_n(m, r, m.size, out)
    return out


def philox4x32_10(ctr, key) -> tuple:
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, np.uint32)
    lib().oracle_philox4x32_10(c, k, out)
    return tuple(int(v) for v in out)


def sr_bits(seed: int, stream: int, e: int) -> int:
    return int(lib().oracle_sr_bits(seed, stream, e))


def sr_bits_n(seed: int, stream: int, e0: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint32)
    lib().oracle_sr_bits_n(seed, stream, e0, n, out)
    return out


def rht_signs_from_seed(seed: int) -> int:
    return int(lib().oracle_rht_signs_from_seed(seed))


# ---------------------------------------------------------------- tensors


@dataclasses.dataclass
class QTensor:
    """An NVFP4 operand [rows, cols] with blocks along cols.

    codes  uint8 [rows, cols/2]  (low nibble = even column)
    scales uint8 E4M3 grid: [rows, cols/16] (mode 0) or [rows/16, cols/16] (mode 1)
    g      float32 decode scale (1 / s_enc)
    """
    codes: np.ndarray
    scales: np.ndarray
    g: np.float32
    rows: int
    cols: int
    mode: int = 0


def _f32(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.float32:
        x = x.astype(np.float32)
    return np.ascontiguousarray(x)


def rht16(x, axis: int, signs: int) -> np.ndarray:
    """Standalone RHT16 of a 2D fp32 matrix along ``axis`` (1 = rows' 16-chunks,
    0 = columns' 16-chunks)  [Review s3]."""
    x = _f32(x)
    R, C = x.shape
    y = np.empty((R, C), np.float32)
    st = lib().oracle_rht16(x, R, C, C, axis, signs, y)
    if st:
        raise OracleError(st)
    return y


def quantize(x, transpose: bool = False, rht: bool = False, signs: int = 0,
             sr: bool = False, seed: int = 0, offset: int = 0, stream: int = 0) -> QTensor:
    """1x16 NVFP4 quantisation of x (or x^T) [Review s1 Steps 1-3, s3, s4]."""
    x = _f32(x)
    sr_, sc_ = x.shape
    R, C = (sc_, sr_) if transpose else (sr_, sc_)
    if C % 16:
        raise OracleError(ERR_SHAPE)
    codes = np.empty((R, C // 2), np.uint8)
    scales = np.empty((R, C // 16), np.uint8)
    g = ctypes.c_float(0.0)
    st = lib().oracle_quantize(x, sr_, sc_, sc_, int(transpose), int(rht), signs, int(sr),
                               seed, offset, stream, codes, scales, ctypes.byref(g))
    if st:
        raise OracleError(st)
    return QTensor(codes, scales, np.float32(g.value), R, C, 0)


def quantize_2d(w, want_t: bool = True):
    """16x16 NVFP4 weight quantisation [Review s2]; returns (W_q, W_q^T or None)."""
    w = _f32(w)
    R, C = w.shape
    if R % 16 or C % 16:
        raise OracleError(ERR_SHAPE)
    codes = np.empty((R, C // 2), np.uint8)
    grid = np.empty((R // 16, C // 16), np.uint8)
    codes_t = np.empty((C, R // 2), np.uint8) if want_t else None
    grid_t = np.empty((C // 16, R // 16), np.uint8) if want_t else None
    g = ctypes.c_float(0.0)
    st = lib().oracle_quantize_2d(
        w, R, C, C, codes, grid,
        codes_t.ctypes.data if want_t else None,
        grid_t.ctypes.data if want_t else None, ctypes.byref(g))
    if st:
        raise OracleError(st)
    q = QTensor(codes, grid, np.float32(g.value), R, C, 1)
    qt = QTensor(codes_t, grid_t, np.float32(g.value), C, R, 1) if want_t else None
    return q, qt


def dequant(q: QTensor) -> np.ndarray:
    """x_hat = decode(code) * d_b * g in float64 [Review s1 Step 3]."""
    out = np.empty((q.rows, q.cols), np.float64)
    lib().oracle_dequant(np.ascontiguousarray(q.codes), np.ascontiguousarray(q.scales),
                         float(q.g), q.rows, q.cols, q.mode, out)
    return out


def gemm(a: QTensor, b: QTensor):
    """C = deq(A) . deq(B)^T and S = |deq(A)| . |deq(B)|^T in float64
    [Review s6; Captions Fig. 5].  The float64 matmul is a library primitive."""
    if a.cols != b.cols:
        raise OracleError(ERR_SHAPE)
    ah, bh = dequant(a), dequant(b)
    return ah @ bh.T, np.abs(ah) @ np.abs(bh).T


def gemm_c(a: QTensor, b: QTensor) -> np.ndarray:
    """C = deq(A) . deq(B)^T alone (the product of gemm() without the
    tolerance sum S)."""
    if a.cols != b.cols:
        raise OracleError(ERR_SHAPE)
    return dequant(a) @ dequant(b).T


def gemm_entries(a_hat: np.ndarray, b_hat: np.ndarray, ms, ns):
    """Selected entries of deq(A) . deq(B)^T, one dot product each."""
    a_hat = np.ascontiguousarray(a_hat, dtype=np.float64)
    b_hat = np.ascontiguousarray(b_hat, dtype=np.float64)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    K = a_hat.shape[1]
    assert b_hat.shape[1] == K and ms.size == ns.size
    c = np.empty(ms.size, np.float64)
    s = np.empty(ms.size, np.float64)
    lib().oracle_gemm_entries(a_hat, b_hat, K, ms, ns, ms.size, c, s)
    return c, s


def dequant_rows(q: QTensor, rows) -> np.ndarray:
    """Dequantise only the listed rows of q (float64 [len(rows), cols])."""
    rows = np.asarray(rows, dtype=np.int64)
    if q.mode == 0:
        sub_scales = q.scales[rows]
        sub = QTensor(q.codes[rows], sub_scales, q.g, rows.size, q.cols, 0)
        return dequant(sub)
    # 16x16 grid: expand the grid rows to per-row scales first
    sub_scales = q.scales[rows // 16]
    sub = QTensor(q.codes[rows], sub_scales, q.g, rows.size, q.cols, 0)
    return dequant(sub)


# ---------------------------------------------------------------- the layer


@dataclasses.dataclass
class Recipe:
    """The pages' training recipe for one linear layer [Review "Core idea"]:
    16x16 weight scales, RHT on the Wgrad inputs only, stochastic rounding on
    the gradient copies only.  Each switch removes one component, as the
    pages' ablations do [Captions Fig. 4, 10, 11, 14]: weights_2d=False
    quantises W (1x16 along K) and W^T (1x16 along N) separately, rht=False
    drops the RHT from the Wgrad copies, sr=False rounds dY to nearest."""
    rht_signs: int
    sr_seed: int = 1234
    weights_2d: bool = True
    rht: bool = True
    sr: bool = True
    # the end-of-training precision switch [Review "Core strengths" item 9;
    # Captions Fig. 7]: Fprop is the plain BF16 product bf16_gemm(x, w); the
    # backward is unchanged
    bf16_fprop: bool = False


def linear_operands(x, w, dy, recipe: Recipe):
    """All six quantised operands of one layer step, Y = X W^T
    [Review s6; Captions Fig. 5]:
      xq   X,  1x16 along K, nearest-even            (Fprop A)
      wq   W,  16x16, nearest-even                   (Fprop B)
      wqt  W^T, the transposed 16x16 copy            (Dgrad B)
      dyq  dY, 1x16 along N, stochastic, stream 0    (Dgrad A)
      dyqt (R dY)^T, RHT along tokens, stochastic, stream 1  (Wgrad A)
      xqt  (R X)^T,  RHT along tokens, nearest-even  (Wgrad B)
    dy may be None (forward only).  With recipe.bf16_fprop the Fprop operands
    xq and wq are not made."""
    s = recipe.rht_signs
    ops = {}
    if not recipe.bf16_fprop:
        ops["xq"] = quantize(x)
    if recipe.weights_2d:
        wq, ops["wqt"] = quantize_2d(w)
        if not recipe.bf16_fprop:
            ops["wq"] = wq
    else:
        if not recipe.bf16_fprop:
            ops["wq"] = quantize(w)
        ops["wqt"] = quantize(w, transpose=True)
    ops["xqt"] = quantize(x, transpose=True, rht=recipe.rht, signs=s)
    if dy is not None:
        ops["dyq"] = quantize(dy, sr=recipe.sr, seed=recipe.sr_seed, stream=0)
        ops["dyqt"] = quantize(dy, transpose=True, rht=recipe.rht, signs=s, sr=recipe.sr,
                               seed=recipe.sr_seed, stream=1)
    return ops


__all__ = [
    "QTensor", "Recipe", "OracleError", "quantize", "quantize_2d", "dequant", "gemm",
    "gemm_entries", "dequant_rows", "rht16", "philox4x32_10", "sr_bits", "sr_bits_n",
    "rht_signs_from_seed", "e2m1_decode", "e4m3_decode", "e4m3_encode",
    "e2m1_rn_index", "e2m1_sr_index", "e4m3_encode_n", "e2m1_rn_index_n",
    "e2m1_sr_index_n", "linear_operands", "lib", "bf16_values", "bf16_gemm",
]


# ---------------------------------------------------------------- MXFP4
# The comparator format [Review "secret weapon" items 1-2; Captions Fig. 6]:
# 32-element blocks, one power-of-two (UE8M0) scale each, no tensor scale.  Scale rule
# (a reading; the pages only describe the format): e = floor(log2(amax_b)) - 2.


@dataclasses.dataclass
class MXTensor:
    """An MXFP4 operand [rows, cols], blocks of 32 along cols."""
    codes: np.ndarray   # uint8 [rows, cols/2], even column in the low nibble
    scales: np.ndarray  # uint8 E8M0 [rows, cols/32]
    rows: int
    cols: int


def e8m0_decode(code: int) -> float:
    return lib().oracle_e8m0_decode(code)


def mx_block(x) -> tuple:
    """One block (<= 32 values) -> (E8M0 scale code, 4-bit codes)."""
    x = _f32(np.asarray(x).reshape(-1))
    codes = np.zeros(x.size, np.uint8)
    sc = lib().oracle_mx_block(x, x.size, codes)
    return int(sc), codes


def mx_quantize(x) -> MXTensor:
    x = _f32(x)
    R, C = x.shape
    codes = np.zeros((R, C // 2), np.uint8)
    scales = np.zeros((R, C // 32), np.uint8)
    st = lib().oracle_mx_quantize(x, R, C, C, codes, scales)
    if st != 0:
        raise OracleError(st)
    return MXTensor(codes, scales, R, C)


def mx_dequant(q: MXTensor) -> np.ndarray:
    out = np.zeros((q.rows, q.cols), np.float64)
    lib().oracle_mx_dequant(np.ascontiguousarray(q.codes), np.ascontiguousarray(q.scales),
                            q.rows, q.cols, out)
    return out


def mx_gemm(a: MXTensor, b: MXTensor):
    """C = deq(A) deq(B)^T in float64 (library matmul over the dequantised
    operands) and S = |deq(A)| |deq(B)|^T for the tolerance."""
    ah, bh = mx_dequant(a), mx_dequant(b)
    return ah @ bh.T, np.abs(ah) @ np.abs(bh).T


# ---------------------------------------------------------------- RHT sizes
# [Review s3 size note; Captions Fig. 12]: d = 4, 16 (the recipe), 128.


def rht_signs128_from_seed(seed: int) -> np.ndarray:
    """The 128 sign bits (4 words, word 0 first, LSB first) from a seed; the
    low 16 bits of word 0 are rht_signs_from_seed(seed)."""
    out = np.zeros(4, np.uint32)
    lib().oracle_rht_signs128_from_seed(seed, out)
    return out


def rht(x, axis: int, d: int, signs) -> np.ndarray:
    """y = fp32(1/sqrt(d)) H_d diag(s) x on every d-element chunk along
    `axis` (1: rows, 0: columns); signs = 4 words of sign bits."""
    x = _f32(x)
    R, C = x.shape
    y = np.empty((R, C), np.float32)
    sg = np.ascontiguousarray(np.asarray(signs, np.uint32).reshape(4))
    st = lib().oracle_rht_d(x, R, C, C, axis, d, sg, y)
    if st:
        raise OracleError(st)
    return y


# ---------------------------------------------------------------- BF16 Fprop
# The high-precision forward of the precision switch [Review "Core strengths"
# item 9; Captions Fig. 7]: Y = X W^T on the bf16 values themselves, no quantisation.


def bf16_values(x) -> np.ndarray:
    """float64 values of bf16 data given as float32 (or float64) numbers;
    raises ValueError for a value bf16 cannot hold (low 16 bits of its fp32
    pattern not zero), so a caller cannot pass unrounded data by mistake."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if np.any(f.view(np.uint32) & 0xFFFF):
        raise ValueError("bf16_values: input not representable in bfloat16")
    return f.astype(np.float64)


def bf16_gemm(a, b):
    """C = A B^T and S = |A| |B|^T in float64 for bf16 A [M, K], B [N, K]
    (the float64 matmul is a library primitive; every product of two bf16
    values is exact in float64)."""
    ah, bh = bf16_values(a), bf16_values(b)
    if ah.ndim != 2 or bh.ndim != 2 or ah.shape[1] != bh.shape[1]:
        raise OracleError(ERR_SHAPE)
    return ah @ bh.T, np.abs(ah) @ np.abs(bh).T
