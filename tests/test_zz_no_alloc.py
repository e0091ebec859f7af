"""nvfp4_quantize_static (no workspace, library-owned reduction slots)
against nvfp4_quantize on the same inputs: codes, block scales and tensor
scale bit for bit, on consecutive calls whose second input is smaller, for
the row copy (nearest and stochastic) and the column copy with the RHT."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import bit_quantized_numerics_amd as nv
    return nv


def _same(a, b, what):
    torch.cuda.synchronize()
    assert (a.rows, a.cols, a.scale_mode) == (b.rows, b.cols, b.scale_mode), what
    assert torch.equal(a.codes_2d(), b.codes_2d()), what + ": codes"
    assert torch.equal(a.scales_2d(), b.scales_2d()), what + ": scales"
    assert a.global_scale.cpu().numpy().tobytes() == b.global_scale.cpu().numpy().tobytes(), \
        what + ": tensor scale"


OPTS = [dict(), dict(round_mode=1, seed=1234, offset=32, stream_id=0),
        dict(transpose=True, rht=True, round_mode=1, seed=99, stream_id=1),
        dict(transpose=True, rht=True)]


@pytest.mark.parametrize("opts", OPTS, ids=["rn", "sr", "col_rht_sr", "col_rht_rn"])
def test_static_matches_workspace_entry_point(nv, opts):
    ws = nv.Workspace("cuda")
    nv.nvfp4_workspace_init(ws)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    signs = nv.nvfp4_rht_signs_from_seed(W.RHT_SEED)
    if opts.get("rht"):
        opts = dict(opts, rht_signs=signs)
    # two calls in a row, the second with a smaller input
    for rows, cols, seed in ((1024, 2560, 1), (272, 400, 2)):
        x = W.activations(rows, cols, seed=seed).cuda()
        say("no-alloc quantise", rows, cols, opts)
        q_static = nv.nvfp4_quantize_static(x, status, **opts)
        q_ws = nv.nvfp4_quantize(x, ws, **opts)
        _same(q_static, q_ws, f"{rows}x{cols} {opts}")
    assert int(status.item()) == nv.OK
    assert nv.nvfp4_device_status(ws) == nv.OK


def test_static_reports_nonfinite_amax(nv):
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    x = torch.ones(64, 256, dtype=torch.bfloat16)
    x[5, 7] = float("inf")
    say("no-alloc quantise, inf input")
    nv.nvfp4_quantize_static(x.cuda(), status)
    torch.cuda.synchronize()
    assert int(status.item()) == nv.ERR_NONFINITE
    # a finite input afterwards uses cleared slots (the status stays raised)
    y = W.activations(64, 256, seed=5).cuda()
    ws = nv.Workspace("cuda")
    nv.nvfp4_workspace_init(ws)
    _same(nv.nvfp4_quantize_static(y, status), nv.nvfp4_quantize(y, ws), "after inf")


def test_static_argument_errors(nv):
    x = torch.zeros(64, 256, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nv.NVFP4Error) as e:
        nv.nvfp4_quantize_static(x, torch.zeros(0, dtype=torch.int32, device="cuda")[:0])
    assert e.value.status in (nv.ERR_NULL, nv.ERR_ALIGN)
    status = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(nv.NVFP4Error) as e:
        nv.nvfp4_quantize_static(x, status.view(torch.uint8)[1:])
    assert e.value.status == nv.ERR_ALIGN
    _ = np
