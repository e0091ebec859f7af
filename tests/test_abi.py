"""CPU tests of the C ABI: the library loads, exports every function
include/nvfp4.h declares, sizes are right, and argument errors are returned
before anything is enqueued (no GPU needed: no call here reaches a launch)."""
import ctypes
import os
import re

import pytest

import bit_quantized_numerics_amd as nv
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "nvfp4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 13
    lib = ctypes.CDLL(nv.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(nv.EXPORTED)


def test_tensor_bytes():
    assert nv.nvfp4_tensor_bytes(64, 256, nv.SCALE_1X16) == (64 * 128, 64 * 16)
    assert nv.nvfp4_tensor_bytes(128, 256, nv.SCALE_16X16) == (128 * 128, 8 * 16)
    for bad in [(64, 24, 0), (0, 16, 0), (24, 32, 1), (16, 16, 5),
                (1 << 40, 1 << 30, 0), ((1 << 62) // 8 + 1, 16, 0)]:   # sizes past 2^62 bytes
        with pytest.raises(nv.NVFP4Error):
            nv.nvfp4_tensor_bytes(*bad)
    assert nv.nvfp4_tensor_bytes(1 << 30, 1 << 20, nv.SCALE_1X16)[0] == (1 << 49)


def test_workspace_bytes_and_status_strings():
    assert nv.nvfp4_workspace_bytes() >= 4096
    for s in range(8):
        assert nv.nvfp4_status_string(s)


def test_rht_signs_from_seed_matches_generator_definition():
    for seed in [0, 1, 1234, 2**40 + 7]:
        assert nv.nvfp4_rht_signs_from_seed(seed) == O.rht_signs_from_seed(seed)


# Fake but non-null, suitably aligned device addresses: every case below must
# be rejected by validation before any HIP call.
P = 1 << 20


def _tensor(codes=P, scales=P, glob=P):
    return nv.c_tensor(codes, scales, glob, 0, 0, 0)


WSB = nv.nvfp4_workspace_bytes()


def _q(x=P, dtype=nv.BF16, rows=64, cols=256, ld=256, opts=None, out=None, ws=P, wsb=WSB):
    o = opts or nv.c_quant_opts(0, 0, 0, 0, 0, 0, 0)
    t = out or _tensor()
    return nv._lib.nvfp4_quantize(x, dtype, rows, cols, ld, ctypes.byref(o), ctypes.byref(t), ws,
                                  wsb, None)


def test_quantize_argument_errors():
    assert _q(x=None) == nv.ERR_NULL
    assert _q(out=_tensor(codes=None)) == nv.ERR_NULL
    assert _q(dtype=7) == nv.ERR_DTYPE
    assert _q(cols=24, ld=24) == nv.ERR_SHAPE
    assert _q(rows=0) == nv.ERR_SHAPE
    assert _q(ld=128) == nv.ERR_SHAPE
    assert _q(rows=65535 * 128 + 16, cols=16, ld=16) == nv.ERR_SHAPE   # row limit
    assert _q(x=P + 2) == nv.ERR_ALIGN
    assert _q(ld=260) == nv.ERR_ALIGN
    assert _q(out=_tensor(codes=P + 4)) == nv.ERR_ALIGN
    assert _q(ws=None) == nv.ERR_WORKSPACE
    assert _q(wsb=WSB - 4) == nv.ERR_WORKSPACE
    assert _q(opts=nv.c_quant_opts(2, 0, 0, 0, 0, 0, 0)) == nv.ERR_DTYPE
    assert _q(opts=nv.c_quant_opts(1, 0, 0, 0, 0, 8, 0)) == nv.ERR_ALIGN       # offset % 16
    assert _q(opts=nv.c_quant_opts(0, 0, 1, 0, 0, 0, 0)) == nv.ERR_SHAPE       # RHT needs transpose
    assert _q(opts=nv.c_quant_opts(0, 1, 1, 0, 0, 0, 0, 8)) == nv.ERR_DTYPE    # RHT size 8
    assert _q(rows=40, opts=nv.c_quant_opts(0, 1, 0, 0, 0, 0, 0)) == nv.ERR_SHAPE
    assert _q(opts=nv.c_quant_opts(0, 1, 1, 0x10000, 0, 0, 0)) == nv.ERR_DTYPE


def test_rowcol_takes_only_the_16_point_transform():
    o_r = nv.c_quant_opts(0, 0, 0, 0, 0, 0, 0)
    o_c = nv.c_quant_opts(0, 1, 1, 0, 0, 0, 1, 4)
    r, c = _tensor(), _tensor()
    assert nv._lib.nvfp4_quantize_rowcol(P, nv.BF16, 64, 256, 256, ctypes.byref(o_r),
                                         ctypes.byref(o_c), ctypes.byref(r), ctypes.byref(c), P,
                                         WSB, None) == nv.ERR_DTYPE
    o_c.rht_d = 16
    assert nv._lib.nvfp4_quantize_rowcol(P, nv.BF16, 64, 256, 256, ctypes.byref(o_r),
                                         ctypes.byref(o_c), ctypes.byref(r), ctypes.byref(c), None,
                                         WSB, None) == nv.ERR_WORKSPACE


def test_gemm_argument_errors():
    a = nv.c_tensor(P, P, P, 64, 256, 0)
    b = nv.c_tensor(P, P, P, 128, 256, 1)
    f = nv._lib.nvfp4_gemm
    assert f(ctypes.byref(a), ctypes.byref(b), None, nv.F32, 128, None, 0, None) == nv.ERR_NULL
    bad_k = nv.c_tensor(P, P, P, 128, 240, 0)
    assert f(ctypes.byref(a), ctypes.byref(bad_k), P, nv.F32, 128, None, 0, None) == nv.ERR_SHAPE
    assert f(ctypes.byref(a), ctypes.byref(b), P, 9, 128, None, 0, None) == nv.ERR_DTYPE
    assert f(ctypes.byref(a), ctypes.byref(b), P, nv.F32, 64, None, 0, None) == nv.ERR_SHAPE
    b2 = nv.c_tensor(P, P, P, 120, 256, 1)  # 16x16 mode needs rows % 16
    assert f(ctypes.byref(a), ctypes.byref(b2), P, nv.F32, 128, None, 0, None) == nv.ERR_SHAPE
    a_mis = nv.c_tensor(P + 8, P, P, 64, 256, 0)
    assert f(ctypes.byref(a_mis), ctypes.byref(b), P, nv.F32, 128, None, 0, None) == nv.ERR_ALIGN


def test_mx_argument_errors():
    """MXFP4 comparator paths: argument errors are caught before any launch."""
    f = nv._lib.nvfp4_gemm
    mx = nv.c_tensor(P, P, None, 64, 512, nv.SCALE_MX32)     # no tensor scale needed
    mx_b = nv.c_tensor(P, P, None, 128, 512, nv.SCALE_MX32)
    nvf = nv.c_tensor(P, P, P, 128, 512, nv.SCALE_1X16)
    assert f(ctypes.byref(mx), ctypes.byref(nvf), P, nv.F32, 128, None, 0, None) == nv.ERR_DTYPE
    small_k = nv.c_tensor(P, P, None, 64, 256, nv.SCALE_MX32)
    small_kb = nv.c_tensor(P, P, None, 128, 256, nv.SCALE_MX32)
    assert f(ctypes.byref(small_k), ctypes.byref(small_kb), P, nv.F32, 128, None, 0,
             None) == nv.ERR_SHAPE
    odd_k = nv.c_tensor(P, P, None, 64, 400, nv.SCALE_MX32)  # cols % 32 != 0
    assert f(ctypes.byref(odd_k), ctypes.byref(mx_b), P, nv.F32, 128, None, 0, None) == nv.ERR_SHAPE
    q = nv._lib.nvfp4_mx_quantize
    out = nv.c_tensor(P, P, None, 0, 0, 0)
    assert q(P, nv.BF16, 64, 48, 48, ctypes.byref(out), None) == nv.ERR_SHAPE  # cols % 32
    assert q(None, nv.BF16, 64, 64, 64, ctypes.byref(out), None) == nv.ERR_NULL
    assert q(P, nv.BF16, 64, 64, 64, None, None) == nv.ERR_NULL
    cb, sb = nv.nvfp4_tensor_bytes(64, 96, nv.SCALE_MX32)
    assert (cb, sb) == (64 * 48, 64 * 3)


def test_dequantize_argument_errors():
    f = nv._lib.nvfp4_dequantize
    t = nv.c_tensor(P, P, P, 64, 256, nv.SCALE_1X16)
    assert f(ctypes.byref(t), None, 256, None) == nv.ERR_NULL
    assert f(ctypes.byref(t), P, 200, None) == nv.ERR_SHAPE       # ldo < cols
    assert f(ctypes.byref(t), P, 258, None) == nv.ERR_SHAPE       # ldo % 4
    assert f(ctypes.byref(t), P + 4, 256, None) == nv.ERR_ALIGN
    no_g = nv.c_tensor(P, P, None, 64, 256, nv.SCALE_1X16)       # NVFP4 needs g
    assert f(ctypes.byref(no_g), P, 256, None) == nv.ERR_NULL


def test_rht_sizes_argument_errors():
    f = nv._lib.nvfp4_rht
    sg = (ctypes.c_uint32 * 4)(0, 0, 0, 0)
    assert f(P, P, nv.BF16, 256, 256, 256, 0, 8, sg, None) == nv.ERR_SHAPE    # d
    assert f(P, P, nv.BF16, 200, 256, 256, 0, 128, sg, None) == nv.ERR_SHAPE  # rows % d
    assert f(P, P, nv.BF16, 256, 100, 100, 1, 4, sg, None) == nv.ERR_SHAPE    # cols % 8
    assert f(P, P, nv.BF16, 256, 256, 256, 0, 128, None, None) == nv.ERR_NULL
    assert f(P, P, 5, 256, 256, 256, 0, 128, sg, None) == nv.ERR_DTYPE
    out = (ctypes.c_uint32 * 4)()
    nv._lib.nvfp4_rht_signs128_from_seed(0, out)
    assert out[0] & 0xFFFF == nv.nvfp4_rht_signs_from_seed(0)


def test_2d_rht_and_layer_argument_errors():
    t = _tensor()
    assert nv._lib.nvfp4_quantize_2d(P, nv.BF16, 40, 32, 32, ctypes.byref(t), None, P, WSB,
                                     None) == nv.ERR_SHAPE
    assert nv._lib.nvfp4_rht16(P, P, nv.F32, 24, 32, 32, 0, 0, None) == nv.ERR_SHAPE
    assert nv._lib.nvfp4_rht16(P, P, nv.F32, 32, 24, 24, 1, 0, None) == nv.ERR_SHAPE
    assert nv._lib.nvfp4_rht16(P, P, nv.F32, 65535 * 128 + 16, 16, 16, 1, 0, None) == nv.ERR_SHAPE
    assert nv._lib.nvfp4_rht16(None, P, nv.F32, 32, 32, 32, 1, 0, None) == nv.ERR_NULL
    assert nv._lib.nvfp4_rht16(P, P, nv.F32, 32, 32, 32, 2, 0, None) == nv.ERR_DTYPE
    rec = nv.c_recipe(0, 1)
    ctx = nv.c_linear_ctx(0, 0, 0, t, t, t, t, t, t)
    assert nv._lib.nvfp4_linear_fwd(P, P, P, 64, 64, 40, nv.BF16, ctypes.byref(rec),
                                    ctypes.byref(ctx), P, WSB, None) == nv.ERR_SHAPE
    assert nv._lib.nvfp4_linear_fwd(P, P, P, 64, 64, 64, nv.BF16, None, ctypes.byref(ctx), P, WSB,
                                    None) == nv.ERR_NULL
    # backward before a training forward on this ctx
    assert nv._lib.nvfp4_linear_bwd(P, nv.BF16, ctypes.byref(ctx), P, P, nv.F32, 1,
                                    ctypes.byref(rec), P, WSB, None) == nv.ERR_SHAPE


def test_bf16_gemm_and_switch_argument_errors():
    f = nv._lib.nvfp4_bf16_gemm
    assert f(None, P, P, 64, 128, 256, nv.F32, 128, None) == nv.ERR_NULL
    assert f(P, P, None, 64, 128, 256, nv.F32, 128, None) == nv.ERR_NULL
    assert f(P, P, P, 64, 128, 256, 7, 128, None) == nv.ERR_DTYPE
    assert f(P, P, P, 64, 128, 64, nv.F32, 128, None) == nv.ERR_SHAPE     # K < 96
    assert f(P, P, P, 64, 128, 272, nv.F32, 128, None) == nv.ERR_SHAPE    # K % 32
    assert f(P, P, P, 0, 128, 256, nv.F32, 128, None) == nv.ERR_SHAPE     # M
    assert f(P, P, P, 64, 128, 256, nv.F32, 100, None) == nv.ERR_SHAPE    # ldc < N
    assert f(P, P, P, 1 << 22, 128, 256, nv.F32, 128, None) == nv.ERR_SHAPE  # 32-bit offsets
    assert f(P + 8, P, P, 64, 128, 256, nv.F32, 128, None) == nv.ERR_ALIGN
    assert f(P, P, P + 2, 64, 128, 256, nv.F32, 128, None) == nv.ERR_ALIGN
    t = _tensor()
    ctx = nv.c_linear_ctx(0, 0, 0, t, t, t, t, t, t)
    rec = nv.c_recipe(0, 1, 0, 0, 0, 1)
    # the BF16 forward needs bf16 inputs and K % 32 == 0
    assert nv._lib.nvfp4_linear_fwd(P, P, P, 64, 256, 64, nv.F32, ctypes.byref(rec),
                                    ctypes.byref(ctx), P, WSB, None) == nv.ERR_DTYPE
    assert nv._lib.nvfp4_linear_fwd(P, P, P, 64, 272, 64, nv.BF16, ctypes.byref(rec),
                                    ctypes.byref(ctx), P, WSB, None) == nv.ERR_SHAPE


def test_linear_ctx_bytes_and_init():
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_linear_ctx_bytes(1 << 40, 1 << 30, 16)   # sizes past 2^62 bytes
    """One-buffer layout of the six layer operands and the backward's split
    scratch (host bookkeeping only)."""
    M, K, N = 64, 96, 160
    nbytes = nv.nvfp4_linear_ctx_bytes(M, K, N)
    a256 = lambda v: (v + 255) // 256 * 256
    shapes = [(M, K), (N, K), (K, N), (K, M), (M, N), (N, M)]
    assert nbytes == sum(a256(r * c // 2) + a256(r * c // 16) + 256
                         for r, c in shapes) + nv.LINEAR_SCRATCH_BYTES
    base = 1 << 24
    ctx = nv.c_linear_ctx()
    assert nv._lib.nvfp4_linear_ctx_init(ctypes.byref(ctx), base, nbytes, M, K, N) == nv.OK
    assert (ctx.M, ctx.K, ctx.N) == (M, K, N)
    end = base
    for name, (r, c) in zip(("xq", "wq", "wqt", "xqt", "dyq", "dyqt"), shapes):
        t = getattr(ctx, name)
        assert (t.rows, t.cols) == (r, c)
        assert t.codes == end and t.codes % 256 == 0
        assert t.scales == t.codes + a256(r * c // 2)
        assert t.global_scale == t.scales + a256(r * c // 16)
        end = t.global_scale + 256
    assert ctx.wgrad_scratch == end and ctx.wgrad_scratch_bytes == nv.LINEAR_SCRATCH_BYTES
    assert end + nv.LINEAR_SCRATCH_BYTES == base + nbytes
    assert (ctx.wq.scale_mode, ctx.xq.scale_mode) == (nv.SCALE_16X16, nv.SCALE_1X16)
    f = nv._lib.nvfp4_linear_ctx_init
    assert f(ctypes.byref(ctx), base, nbytes - 1, M, K, N) == nv.ERR_SHAPE
    assert f(ctypes.byref(ctx), base + 16, nbytes, M, K, N) == nv.ERR_ALIGN
    assert f(ctypes.byref(ctx), None, nbytes, M, K, N) == nv.ERR_NULL
    assert f(ctypes.byref(ctx), base, nbytes, M, K, 40) == nv.ERR_SHAPE
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_linear_ctx_bytes(0, K, N)


def test_peak_helper_argument_errors():
    flops = ctypes.c_double(0)
    f = nv._lib.nvfp4_peak_mfma_f16
    assert f(100, 0, 4, None, ctypes.byref(flops), None) == nv.ERR_NULL
    assert f(100, 0, 4, P, None, None) == nv.ERR_NULL
    assert f(0, 0, 4, P, ctypes.byref(flops), None) == nv.ERR_SHAPE
    assert f(100, 0, 2, P, ctypes.byref(flops), None) == nv.ERR_DTYPE
    g = nv._lib.nvfp4_peak_mfma_fp4
    assert g(100, 0, None, ctypes.byref(flops), None) == nv.ERR_NULL
    assert g(100, 0, P, None, None) == nv.ERR_NULL
    assert g(-1, 0, P, ctypes.byref(flops), None) == nv.ERR_SHAPE


def test_quantize_static_argument_errors():
    """Argument errors of the allocation-free variant come back before any
    HIP call (and so before the per-device scratch is looked up)."""
    f = nv._lib.nvfp4_quantize_static
    o = nv.c_quant_opts(0, 0, 0, 0, 0, 0, 0)
    t = _tensor()
    assert f(None, nv.BF16, 64, 256, 256, ctypes.byref(o), ctypes.byref(t), P, None) == nv.ERR_NULL
    assert f(P, nv.BF16, 64, 256, 256, ctypes.byref(o), ctypes.byref(t), None, None) == nv.ERR_NULL
    assert f(P, nv.BF16, 64, 256, 256, ctypes.byref(o), ctypes.byref(t), P + 2, None) == nv.ERR_ALIGN
    assert f(P, nv.BF16, 64, 24, 24, ctypes.byref(o), ctypes.byref(t), P, None) == nv.ERR_SHAPE
    bad = nv.c_quant_opts(0, 0, 1, 0, 0, 0, 0)   # RHT without transpose
    assert f(P, nv.BF16, 64, 256, 256, ctypes.byref(bad), ctypes.byref(t), P, None) == nv.ERR_SHAPE


def test_backward_refuses_another_rht_than_its_forward():
    """The Wgrad operands (R dY)^T and (R X)^T need one transform: a backward
    recipe with other signs, or with the RHT switched on or off against the
    forward's, is refused before anything is enqueued."""
    M, K, N = 64, 96, 160
    ctx = nv.c_linear_ctx()
    nbytes = nv.nvfp4_linear_ctx_bytes(M, K, N)
    assert nv._lib.nvfp4_linear_ctx_init(ctypes.byref(ctx), P, nbytes, M, K, N) == nv.OK
    assert (ctx.rht_signs, ctx.rht) == (0, 0)
    ctx.rht_signs, ctx.rht = 0x1234, 1          # what a training forward records
    bwd = nv._lib.nvfp4_linear_bwd
    for rec, want in ((nv.c_recipe(0x1235, 1), nv.ERR_SHAPE),           # other signs
                      (nv.c_recipe(0x1234, 1, 0, 1), nv.ERR_SHAPE),      # RHT off
                      (nv.c_recipe(0x1234, 1), nv.ERR_WORKSPACE)):       # matches: next check
        assert bwd(P, nv.BF16, ctypes.byref(ctx), P, P, nv.F32, 1, ctypes.byref(rec), None, 0,
                   None) == want
    ctx.rht = 0                                 # forward ran with no_rht
    assert bwd(P, nv.BF16, ctypes.byref(ctx), P, P, nv.F32, 1, ctypes.byref(nv.c_recipe(0x1234, 1)),
               None, 0, None) == nv.ERR_SHAPE
    assert bwd(P, nv.BF16, ctypes.byref(ctx), P, P, nv.F32, 1,
               ctypes.byref(nv.c_recipe(0x1234, 1, 0, 1)), None, 0, None) == nv.ERR_WORKSPACE
