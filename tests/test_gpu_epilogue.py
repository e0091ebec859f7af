"""GPU parity of the GEMM epilogue (scaling, bf16 rounding, the quad
transpose and the store paths) for every GEMM family: the product is written
into a column window of a wider buffer filled with a sentinel, and nothing
outside the window may change.

Two window layouts: "aligned" (row stride a multiple of 4 elements, base
aligned, N % 4 = 2, so the vector stores and the ragged last quad both run)
and "offset" (base moved by 2 elements and an odd row stride, so every store
takes the per-element path).  M is not a multiple of 32 either."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests.gpu_util import assert_gemm_close, np32, say

pytestmark = pytest.mark.gpu

M, N = 70, 50
SENTINEL = 7.0


@pytest.fixture(scope="module")
def nv():
    import bit_quantized_numerics_amd as nv
    return nv


@pytest.fixture(scope="module")
def ws(nv):
    w = nv.Workspace("cuda")
    nv.nvfp4_workspace_init(w)
    return w


def _window(layout, out):
    if layout == "aligned":
        big = torch.full((M, 64), SENTINEL, dtype=out, device="cuda")
        return big, 0
    big = torch.full((M, N + 9), SENTINEL, dtype=out, device="cuda")  # row stride 59
    return big, 2


# family, K: K = 272 takes the NVFP4 direct kernel, 384 the 128-k slab kernel,
# 512 the 256-k slab kernel; the MXFP4 and BF16 GEMMs take their wide kernels.
CASES = [("nvfp4", 272), ("nvfp4", 384), ("nvfp4", 512), ("mx", 512), ("bf16", 256)]


@pytest.mark.parametrize("layout", ["aligned", "offset"])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("family,K", CASES)
def test_output_window(nv, ws, family, K, out, layout):
    a = W.activations(M, K, seed=W.SEED_X + 70 + K)
    b = W.weights(N, K, seed=W.SEED_W + 70 + K)
    big, off = _window(layout, out)
    c = big[:, off:off + N]
    say("epilogue", family, K, out, layout)
    if family == "nvfp4":
        nv.nvfp4_gemm(nv.nvfp4_quantize(a.cuda(), ws), nv.nvfp4_quantize(b.cuda(), ws), c=c)
        C, S = O.gemm(O.quantize(np32(a)), O.quantize(np32(b)))
    elif family == "mx":
        nv.nvfp4_gemm(nv.nvfp4_mx_quantize(a.cuda()), nv.nvfp4_mx_quantize(b.cuda()), c=c)
        C, S = O.mx_gemm(O.mx_quantize(np32(a)), O.mx_quantize(np32(b)))
    else:
        nv.nvfp4_bf16_gemm(a.cuda(), b.cuda(), c=c)
        C, S = O.bf16_gemm(np32(a), np32(b))
    torch.cuda.synchronize()
    got = big.float().cpu().numpy()
    assert_gemm_close(got[:, off:off + N], C, S, out == torch.bfloat16, f"{family} K={K} {layout}")
    outside = np.ones(got.shape, bool)
    outside[:, off:off + N] = False
    assert np.all(got[outside] == SENTINEL)
