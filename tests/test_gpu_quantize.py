"""GPU parity of the quantisers and the standalone RHT against the oracle:
codes, E4M3 block scales and the FP32 tensor scale must agree bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests.gpu_util import assert_q_equal, np32, say

pytestmark = pytest.mark.gpu

SIGNS = O.rht_signs_from_seed(W.RHT_SEED)


@pytest.fixture(scope="module")
def nv():
    import bit_quantized_numerics_amd as nv
    return nv


@pytest.fixture()
def ws(nv):
    w = nv.Workspace("cuda")
    nv.nvfp4_workspace_init(w)
    return w


def _rand(rows, cols, dtype, seed, p=0.01, mul=30.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, cols, generator=g)
    m = torch.rand(rows, cols, generator=g) < p
    x[m] *= mul
    return x.to(dtype)


SHAPES = [(64, 256, torch.float32), (37, 48, torch.bfloat16), (272, 400, torch.bfloat16),
          (512, 1024, torch.bfloat16), (16, 16, torch.float32)]


@pytest.mark.parametrize("rows,cols,dtype", SHAPES)
@pytest.mark.parametrize("sr", [False, True])
def test_row_quantize(nv, ws, rows, cols, dtype, sr):
    x = _rand(rows, cols, dtype, rows * 7 + cols)
    say("row", rows, cols, dtype, sr)
    q = nv.nvfp4_quantize(x.cuda(), ws, round_mode=nv.SR if sr else nv.RN, seed=1234,
                          offset=32 if sr else 0, stream_id=5 if sr else 0)
    ref = O.quantize(np32(x), sr=sr, seed=1234, offset=32 if sr else 0, stream=5 if sr else 0)
    assert_q_equal(q, ref, "row")
    assert nv.nvfp4_device_status(ws) == nv.OK


COL_SHAPES = [(64, 256, torch.float32), (272, 400, torch.bfloat16), (1024, 384, torch.bfloat16),
              (48, 32, torch.float32)]


@pytest.mark.parametrize("rows,cols,dtype", COL_SHAPES)
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("rht", [False, True])
def test_col_quantize(nv, ws, rows, cols, dtype, sr, rht):
    x = _rand(rows, cols, dtype, rows * 3 + cols)
    say("col", rows, cols, dtype, sr, rht)
    q = nv.nvfp4_quantize(x.cuda(), ws, round_mode=nv.SR if sr else nv.RN, transpose=True, rht=rht,
                          rht_signs=SIGNS, seed=99, offset=16, stream_id=1)
    ref = O.quantize(np32(x), transpose=True, rht=rht, signs=SIGNS, sr=sr, seed=99, offset=16,
                     stream=1)
    assert_q_equal(q, ref, "col")


@pytest.mark.parametrize("rows,cols,dtype", [(272, 400, torch.bfloat16), (512, 1024, torch.float32),
                                             (64, 256, torch.float32)])
@pytest.mark.parametrize("sr_row,sr_col,rht", [(False, False, True), (True, True, True),
                                               (True, False, False), (False, True, False)])
def test_rowcol_quantize(nv, ws, rows, cols, dtype, sr_row, sr_col, rht):
    x = _rand(rows, cols, dtype, rows + cols * 5)
    say("rowcol", rows, cols, dtype, sr_row, sr_col, rht)
    r, c = nv.nvfp4_quantize_rowcol(x.cuda(), ws, round_row=nv.SR if sr_row else nv.RN,
                                    round_col=nv.SR if sr_col else nv.RN, rht=rht, rht_signs=SIGNS,
                                    seed=1234)
    xr = np32(x)
    assert_q_equal(r, O.quantize(xr, sr=sr_row, seed=1234, stream=0), "rowcol/row")
    assert_q_equal(c, O.quantize(xr, transpose=True, rht=rht, signs=SIGNS, sr=sr_col, seed=1234,
                                 stream=1), "rowcol/col")


@pytest.mark.parametrize("rows,cols,dtype", [(128, 256, torch.float32), (272, 400, torch.bfloat16),
                                             (1024, 768, torch.bfloat16), (16, 16, torch.float32)])
def test_quantize_2d(nv, ws, rows, cols, dtype):
    w = (_rand(rows, cols, dtype, rows + cols, p=0.05).float() * 0.02).to(dtype)
    say("2d", rows, cols, dtype)
    q, qt = nv.nvfp4_quantize_2d(w.cuda(), ws)
    ref, ref_t = O.quantize_2d(np32(w))
    assert_q_equal(q, ref, "2d")
    assert_q_equal(qt, ref_t, "2d/t")
    q2, none = nv.nvfp4_quantize_2d(w.cuda(), ws, want_t=False)
    assert none is None
    assert_q_equal(q2, ref, "2d without transpose")


def test_zero_and_degenerate_inputs(nv, ws):
    z = torch.zeros(32, 64, dtype=torch.bfloat16)
    say("zeros")
    q = nv.nvfp4_quantize(z.cuda(), ws)
    assert_q_equal(q, O.quantize(np32(z)), "zeros")
    x = _rand(32, 64, torch.float32, 5)
    x[:, :16] = 0.0
    x[3, 20] = -0.0
    x[5, 40:56] = 1e-30
    say("zero blocks")
    r, c = nv.nvfp4_quantize_rowcol(x.cuda(), ws, rht=True, rht_signs=SIGNS)
    assert_q_equal(r, O.quantize(np32(x)), "zero blocks row")
    assert_q_equal(c, O.quantize(np32(x), transpose=True, rht=True, signs=SIGNS), "zero blocks col")
    tiny = torch.zeros(16, 16)
    tiny[0, 0] = 1e-39
    tiny[1, 1] = -3e-40
    say("subnormal amax")
    q = nv.nvfp4_quantize(tiny.cuda(), ws)
    assert_q_equal(q, O.quantize(np32(tiny)), "subnormal amax")
    assert nv.nvfp4_device_status(ws) == nv.OK


@pytest.mark.parametrize("bad", [float("inf"), float("nan"), -float("inf")])
def test_nonfinite_sets_device_status(nv, ws, bad):
    x = _rand(32, 64, torch.float32, 6)
    x[7, 9] = bad
    say("nonfinite", bad)
    nv.nvfp4_quantize(x.cuda(), ws)
    assert nv.nvfp4_device_status(ws) == nv.ERR_NONFINITE
    assert nv.nvfp4_device_status(ws) == nv.OK  # reading clears it
    nv.nvfp4_quantize_2d(x.cuda(), ws)
    assert nv.nvfp4_device_status(ws) == nv.ERR_NONFINITE
    with pytest.raises(O.OracleError):
        O.quantize(np32(x))


def test_determinism(nv, ws):
    x = _rand(512, 1024, torch.bfloat16, 8).cuda()
    say("determinism")
    a = nv.nvfp4_quantize_rowcol(x, ws, round_row=nv.SR, round_col=nv.SR, rht=True, rht_signs=SIGNS,
                                 seed=7)
    b = nv.nvfp4_quantize_rowcol(x, ws, round_row=nv.SR, round_col=nv.SR, rht=True, rht_signs=SIGNS,
                                 seed=7)
    for u, v in zip(a, b):
        assert torch.equal(u.codes, v.codes) and torch.equal(u.scales, v.scales)
    c = nv.nvfp4_quantize_rowcol(x, ws, round_row=nv.SR, round_col=nv.SR, rht=True, rht_signs=SIGNS,
                                 seed=8)
    assert not torch.equal(a[0].codes, c[0].codes)


@pytest.mark.parametrize("rows,cols,dtype", [(64, 256, torch.float32), (272, 400, torch.bfloat16),
                                             (1024, 768, torch.bfloat16)])
@pytest.mark.parametrize("axis", [0, 1])
def test_rht16(nv, rows, cols, dtype, axis):
    x = _rand(rows, cols, dtype, rows ^ cols)
    say("rht16", rows, cols, dtype, axis)
    y = nv.nvfp4_rht16(x.cuda(), axis, SIGNS)
    ref = O.rht16(np32(x), axis, SIGNS)
    got = y.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------ full layer shapes


@pytest.mark.slow
def test_full_size_x_rowcol(nv, ws):
    x = W.activations(W.LAYER_M, W.LAYER_K)
    say("full X rowcol", tuple(x.shape))
    r, c = nv.nvfp4_quantize_rowcol(x.cuda(), ws, rht=True, rht_signs=SIGNS)
    xr = np32(x)
    assert_q_equal(r, O.quantize(xr), "X row")
    assert_q_equal(c, O.quantize(xr, transpose=True, rht=True, signs=SIGNS), "X col")


@pytest.mark.slow
def test_full_size_dy_rowcol_sr(nv, ws):
    dy = W.gradients(W.LAYER_M, W.LAYER_N)
    say("full dY rowcol SR", tuple(dy.shape))
    r, c = nv.nvfp4_quantize_rowcol(dy.cuda(), ws, round_row=nv.SR, round_col=nv.SR, rht=True,
                                    rht_signs=SIGNS, seed=W.SR_SEED)
    dr = np32(dy)
    del dy
    assert_q_equal(r, O.quantize(dr, sr=True, seed=W.SR_SEED, stream=0), "dY row")
    assert_q_equal(c, O.quantize(dr, transpose=True, rht=True, signs=SIGNS, sr=True,
                                 seed=W.SR_SEED, stream=1), "dY col")


@pytest.mark.slow
def test_full_size_w_2d(nv, ws):
    w = W.weights(W.LAYER_N, W.LAYER_K)
    say("full W 2d", tuple(w.shape))
    q, qt = nv.nvfp4_quantize_2d(w.cuda(), ws)
    ref, ref_t = O.quantize_2d(np32(w))
    assert_q_equal(q, ref, "W")
    assert_q_equal(qt, ref_t, "W^T")


@pytest.mark.parametrize("scale_log2", [-140, -126, -100, 0, 90, 93, 96, 99, 110])
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("d", [16, 4])
def test_col_rht_across_magnitudes(nv, ws, scale_log2, sr, d):
    """Column copies with the RHT of bf16 data scaled by 2^k across the whole
    range: tiny values whose transform lands in fp32's subnormal range, and
    huge ones around the 2^100 amax below which the kernel folds the
    transform's final 1/4 (or 1/2) into the multiplier.  Codes, scales and
    tensor scale must equal the oracle's (separate transform, then
    quantisation) in every case."""
    x = (_rand(256, 384, torch.float32, 40 + scale_log2 & 0xFF, p=0.02, mul=20.0) *
         2.0 ** scale_log2).to(torch.bfloat16)
    x[3, :16] = 0.0
    x[9, 5] = -0.0
    xr = np32(x)
    say("col rht magnitudes", scale_log2, sr, d)
    q = nv.nvfp4_quantize(x.cuda(), ws, transpose=True, rht=True, rht_d=d, rht_signs=SIGNS,
                          round_mode=nv.SR if sr else nv.RN, seed=77, stream_id=1)
    if d == 16:
        ref = O.quantize(xr, transpose=True, rht=True, signs=SIGNS, sr=sr, seed=77, stream=1)
    else:
        sg = [SIGNS & 0xF, 0, 0, 0]
        ref = O.quantize(O.rht(xr, 0, 4, sg), transpose=True, sr=sr, seed=77, stream=1)
    assert nv.nvfp4_device_status(ws) == nv.OK
    assert_q_equal(q, ref, f"col rht d={d} 2^{scale_log2}")
