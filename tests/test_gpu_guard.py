"""Reads stay inside each operand.  Every source or GEMM operand here is the
leading rows of a larger device buffer whose trailing rows hold values that
would change the result if a kernel read them (huge values, NaN, the largest
codes and scales).  Rows past an operand must read as absent: a quantiser's
tensor amax, block scales and codes, and a GEMM's stored outputs, must equal
the oracle's on the operand alone, and no non-finite status may appear.  The
trailing rows are inside the allocation, so a kernel that did read them
returns a wrong answer instead of faulting."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests.gpu_util import assert_gemm_close, assert_q_equal, np32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import bit_quantized_numerics_amd as nv
    return nv


@pytest.fixture()
def ws(nv):
    w = nv.Workspace("cuda")
    nv.nvfp4_workspace_init(w)
    return w


def _guarded(rows, cols, dtype, seed, poison, extra=272):
    """A [rows, cols] view of the first rows of a [rows + extra, cols] device
    buffer whose trailing rows are `poison`."""
    g = torch.Generator().manual_seed(seed)
    full = torch.randn(rows + extra, cols, generator=g)
    full[rows:] = poison
    full = full.to(dtype).cuda()
    return full[:rows], np32(full[:rows])


@pytest.mark.parametrize("rows", [1, 37, 129, 300])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("poison", [1e30, float("nan")])
@pytest.mark.parametrize("sr", [False, True])
def test_quantize_ragged_rows_guard(nv, ws, rows, dtype, poison, sr):
    cols = 272
    x, xr = _guarded(rows, cols, dtype, rows + 11, poison)
    say("guard quantize", rows, cols, dtype, poison, sr)
    q = nv.nvfp4_quantize(x, ws, round_mode=nv.SR if sr else nv.RN, seed=7)
    assert nv.nvfp4_device_status(ws) == nv.OK
    assert_q_equal(q, O.quantize(xr, sr=sr, seed=7), "guarded row copy")


@pytest.mark.parametrize("rows", [16, 144, 272])
@pytest.mark.parametrize("poison", [1e30, float("nan")])
def test_quantize_columns_guard(nv, ws, rows, poison):
    """Column copies (rows % 16 == 0, RHT along tokens) with poisoned rows after."""
    cols = 400
    x, xr = _guarded(rows, cols, torch.bfloat16, rows + 5, poison)
    signs = O.rht_signs_from_seed(W.RHT_SEED)
    say("guard rowcol", rows, cols, poison)
    r, c = nv.nvfp4_quantize_rowcol(x, ws, round_row=nv.SR, round_col=nv.SR, rht=True,
                                    rht_signs=signs, seed=3)
    assert nv.nvfp4_device_status(ws) == nv.OK
    assert_q_equal(r, O.quantize(xr, sr=True, seed=3, stream=0), "guarded row")
    assert_q_equal(c, O.quantize(xr, transpose=True, rht=True, signs=signs, sr=True, seed=3,
                                 stream=1), "guarded col")
    w2, w2t = nv.nvfp4_quantize_2d(x, ws)
    assert nv.nvfp4_device_status(ws) == nv.OK
    r2, r2t = O.quantize_2d(xr)
    assert_q_equal(w2, r2, "guarded 2d")
    assert_q_equal(w2t, r2t, "guarded 2d^T")


@pytest.mark.parametrize("rows", [1, 37, 300])
def test_mx_quantize_ragged_rows_guard(nv, rows):
    x, xr = _guarded(rows, 256, torch.bfloat16, rows, float("nan"))
    say("guard mx quantize", rows)
    q = nv.nvfp4_mx_quantize(x)
    torch.cuda.synchronize()
    ref = O.mx_quantize(xr)
    assert np.array_equal(q.codes_2d().cpu().numpy(), ref.codes)
    assert np.array_equal(q.scales_2d().cpu().numpy(), ref.scales)


def _poisoned_copy(nv, q, code_byte, scale_byte, extra_rows=272):
    """The operand q copied into buffers with `extra_rows` poisoned rows after it."""
    t = nv.NVFP4Tensor(q.rows + extra_rows, q.cols, q.scale_mode, device="cuda")
    t.codes.fill_(code_byte)
    t.scales.fill_(scale_byte)
    nc, ns = q.codes_2d().numel(), q.scales_2d().numel()
    t.codes[:nc].copy_(q.codes[:nc])
    t.scales[:ns].copy_(q.scales[:ns])
    t.global_scale.copy_(q.global_scale)
    t.rows = q.rows
    return t


@pytest.mark.parametrize("M,N,K", [(300, 130, 768), (37, 520, 512), (257, 257, 1536),
                                   (300, 130, 400)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_gemm_operand_tail_guard(nv, ws, M, N, K, out):
    """GEMM operands whose buffers continue with code 0x77 (+6, +6) and scale
    0x7F (E4M3 NaN) / 0x7E (448): only the operand's own rows may count."""
    g = torch.Generator().manual_seed(M + N + K)
    a = torch.randn(M, K, generator=g)
    b = torch.randn(N, K, generator=g)
    say("guard gemm", M, N, K, out)
    qa = nv.nvfp4_quantize(a.cuda(), ws)
    qb = nv.nvfp4_quantize(b.cuda(), ws)
    ga = _poisoned_copy(nv, qa, 0x77, 0x7F)
    gb = _poisoned_copy(nv, qb, 0x77, 0x7E)
    c = nv.nvfp4_gemm(ga, gb, out)
    C, S = O.gemm(O.quantize(a.numpy()), O.quantize(b.numpy()))
    assert_gemm_close(c.float().cpu().numpy(), C, S, out == torch.bfloat16, "guarded gemm")


@pytest.mark.parametrize("M,N", [(300, 130), (37, 520)])
def test_mx_gemm_operand_tail_guard(nv, M, N):
    K = 768
    g = torch.Generator().manual_seed(M * N)
    a = torch.randn(M, K, generator=g)
    b = torch.randn(N, K, generator=g)
    say("guard mx gemm", M, N, K)
    qa = nv.nvfp4_mx_quantize(a.cuda())
    qb = nv.nvfp4_mx_quantize(b.cuda())
    ga = _poisoned_copy(nv, qa, 0x77, 0xFF)
    gb = _poisoned_copy(nv, qb, 0x77, 0xFE)
    c = nv.nvfp4_gemm(ga, gb, torch.float32)
    C, S = O.mx_gemm(O.mx_quantize(a.numpy()), O.mx_quantize(b.numpy()))
    assert_gemm_close(c.cpu().numpy(), C, S, False, "guarded mx gemm")


@pytest.mark.parametrize("M,N", [(300, 130), (37, 520)])
def test_bf16_gemm_operand_tail_guard(nv, M, N):
    K = 512
    g = torch.Generator().manual_seed(M + 3 * N)
    fa = torch.randn(M + 272, K, generator=g)
    fb = torch.randn(N + 272, K, generator=g)
    fa[M:] = float("nan")
    fb[N:] = float("inf")
    fa, fb = fa.to(torch.bfloat16).cuda(), fb.to(torch.bfloat16).cuda()
    say("guard bf16 gemm", M, N, K)
    c = nv.nvfp4_bf16_gemm(fa[:M], fb[:N], torch.float32)
    C, S = O.bf16_gemm(np32(fa[:M]), np32(fb[:N]))
    assert_gemm_close(c.cpu().numpy(), C, S, False, "guarded bf16 gemm")
