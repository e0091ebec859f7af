"""GPU parity of nvfp4_rht (Hadamard sizes 4, 16, 128 and the sign options)
against the oracle, bit for bit (same fp32 operation order), and of a Wgrad
operand built with the 128-point transform: nvfp4_rht along tokens then
nvfp4_quantize of the transpose, against the oracle's composition."""
import numpy as np
import pytest
import torch

import oracle as O
from tests.gpu_util import assert_q_equal, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import bit_quantized_numerics_amd as nv
    return nv


@pytest.mark.parametrize("d", [4, 16, 128])
@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("seed", [0, 41])
def test_rht_sizes(nv, d, axis, dtype, seed):
    g = torch.Generator().manual_seed(d * 7 + axis)
    x = (torch.randn(256, 384, generator=g) * 3.0).to(dtype)
    signs = nv.nvfp4_rht_signs128_from_seed(seed)
    assert list(signs) == [int(v) for v in O.rht_signs128_from_seed(seed)]
    say("rht", d, axis, dtype, seed)
    y = nv.nvfp4_rht(x.cuda(), axis, d, signs).cpu().numpy()
    ref = O.rht(x.float().numpy(), axis, d, np.array(signs, np.uint32))
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32)), \
        f"{np.count_nonzero(y != ref)} values differ"


@pytest.mark.parametrize("d", [4, 128])
def test_no_randomisation(nv, d):
    x = torch.eye(d, dtype=torch.float32)
    y = nv.nvfp4_rht(x.cuda(), 0, d, (0, 0, 0, 0)).cpu().numpy()
    ref = O.rht(x.numpy(), 0, d, np.zeros(4, np.uint32))
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("d", [4, 128])
def test_wgrad_operand_with_other_size(nv, d):
    """(R_d X)^T quantised along tokens: transform then quantise the transpose."""
    g = torch.Generator().manual_seed(5)
    M, K = 512, 192
    x = torch.randn(M, K, generator=g).to(torch.bfloat16)
    signs = nv.nvfp4_rht_signs128_from_seed(3)
    ws = nv.Workspace("cuda")
    nv.nvfp4_workspace_init(ws)
    say("wgrad operand rht", d)
    y = nv.nvfp4_rht(x.cuda(), 0, d, signs)
    q = nv.nvfp4_quantize(y, ws, transpose=True)
    ref = O.quantize(O.rht(x.float().numpy(), 0, d, np.array(signs, np.uint32)), transpose=True)
    assert_q_equal(q, ref, f"wgrad operand d={d}")


# (rows, cols): several 128-row emit tiles with a ragged column tile; a single
# 16-token chunk row; odd tile counts.
@pytest.mark.parametrize("rows,cols", [(512, 400), (16, 256), (272, 48)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("sr", [False, True])
def test_fused_d4_quantise(nv, rows, cols, dtype, sr):
    """The 4-point transform fused into the quantiser (rht_d = 4): equal, code
    for code, to the oracle's separate 4-point transform along tokens followed
    by its quantisation of the transpose (the fused kernel computes the same
    fp32 values in registers)."""
    g = torch.Generator().manual_seed(rows + cols)
    x = (torch.randn(rows, cols, generator=g) * 2.0).to(dtype)
    x[0, :] *= 40.0  # an outlier row
    signs = nv.nvfp4_rht_signs128_from_seed(7)
    s16 = int(signs[0]) & 0xFFFF
    ws = nv.Workspace("cuda")
    nv.nvfp4_workspace_init(ws)
    say("fused d4", rows, cols, dtype, sr)
    q = nv.nvfp4_quantize(x.cuda(), ws, transpose=True, rht=True, rht_d=4, rht_signs=s16,
                          round_mode=nv.SR if sr else nv.RN, seed=1234, stream_id=1)
    y = O.rht(x.float().numpy(), 0, 4, np.array(signs, np.uint32))
    ref = O.quantize(y, transpose=True, sr=sr, seed=1234, stream=1)
    assert_q_equal(q, ref, f"fused d4 {rows}x{cols} {dtype} sr={sr}")
    assert nv.nvfp4_device_status(ws) == nv.OK
