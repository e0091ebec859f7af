"""GPU parity of the BF16 forward of the precision switch [Review "Core
strengths" item 9; Captions Fig. 7]: nvfp4_bf16_gemm against the oracle's float64 product of
the same bf16 values, and nvfp4_linear_fwd with bf16_fprop (Y from the BF16
product, the backward copies bit-exact against the oracle and the backward
unchanged bit for bit)."""
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


# (M, N, K): one slab-triple minimum K, ragged M and N, several 256 x 256
# tiles, a long K, a single output element.
SHAPES = [(256, 256, 96), (100, 130, 128), (528, 400, 640), (300, 1000, 3200), (1, 1, 96),
          (17, 300, 4096)]


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_bf16_gemm(nv, M, N, K, out):
    a = W.activations(M, K, seed=W.SEED_X + 40)
    b = W.weights(N, K, seed=W.SEED_W + 40)
    say("bf16 gemm", M, N, K, out)
    c = nv.nvfp4_bf16_gemm(a.cuda(), b.cuda(), out)
    torch.cuda.synchronize()
    C, S = O.bf16_gemm(np32(a), np32(b))
    assert_gemm_close(c.float().cpu().numpy(), C, S, out == torch.bfloat16, f"bf16 {M}x{N}x{K}")


def test_bf16_gemm_exact_integers(nv):
    """Small integers: every partial sum is exact in fp32, so the result must
    equal the oracle bit for bit whatever the accumulation order."""
    g = torch.Generator().manual_seed(41)
    M, N, K = 384, 320, 1024
    a = torch.randint(-3, 4, (M, K), generator=g).to(torch.bfloat16)
    b = torch.randint(-3, 4, (N, K), generator=g).to(torch.bfloat16)
    say("bf16 gemm exact", M, N, K)
    c = nv.nvfp4_bf16_gemm(a.cuda(), b.cuda(), torch.float32).cpu().numpy()
    C, _ = O.bf16_gemm(np32(a), np32(b))
    assert np.array_equal(c.astype(np.float64), C)


def test_bf16_gemm_output_stride(nv):
    """ldc > N: the product lands in a column window of a wider buffer and
    nothing outside it is written."""
    M, N, K = 130, 200, 256
    a = W.activations(M, K, seed=W.SEED_X + 42)
    b = W.weights(N, K, seed=W.SEED_W + 42)
    big = torch.full((M, N + 72), 7.0, dtype=torch.float32, device="cuda")
    say("bf16 gemm ldc", M, N, K)
    nv.nvfp4_bf16_gemm(a.cuda(), b.cuda(), torch.float32, c=big[:, :N])
    torch.cuda.synchronize()
    C, S = O.bf16_gemm(np32(a), np32(b))
    got = big.cpu().numpy()
    assert_gemm_close(got[:, :N], C, S, False, "bf16 ldc")
    assert np.all(got[:, N:] == 7.0)


@pytest.mark.slow
def test_bf16_gemm_full_size_sampled(nv):
    """The layer's Fprop shape X [8192, 5120] x W [20480, 5120] -> Y bf16."""
    M, K, N = 8192, 5120, 20480
    x = W.activations(M, K)
    w = W.weights(N, K)
    say("bf16 gemm full", M, N, K)
    y = nv.nvfp4_bf16_gemm(x.cuda(), w.cuda(), torch.bfloat16)
    torch.cuda.synchronize()
    g = np.random.default_rng(3)
    ms = np.concatenate([g.integers(0, M, 384), [0, M - 1, 0, M - 1]])
    ns = np.concatenate([g.integers(0, N, 384), [0, N - 1, N - 1, 0]])
    um, im = np.unique(ms, return_inverse=True)
    un, in_ = np.unique(ns, return_inverse=True)
    a_rows = O.bf16_values(np32(x[torch.from_numpy(um)]))
    b_rows = O.bf16_values(np32(w[torch.from_numpy(un)]))
    Cs, Ss = O.gemm_entries(a_rows, b_rows, im, in_)
    got = y[torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()].float().cpu().numpy()
    assert_gemm_close(got, Cs, Ss, True, "bf16 full")


@pytest.mark.parametrize("two_d", [True, False], ids=["2d", "1x16"])
@pytest.mark.parametrize("M,K,N", [(256, 384, 512), (512, 2048, 512)])
def test_layer_bf16_fprop(nv, two_d, M, K, N):
    x = W.activations(M, K, seed=W.SEED_X + 43)
    w = W.weights(N, K, seed=W.SEED_W + 43)
    dy = W.gradients(M, N, seed=W.SEED_DY + 43)
    signs = nv.nvfp4_rht_signs_from_seed(W.RHT_SEED)
    ws = nv.Workspace("cuda")
    nv.nvfp4_workspace_init(ws)
    sw = dict(no_2d_weights=not two_d)
    xc, wc, dyc = x.cuda(), w.cuda(), dy.cuda()
    say("layer bf16 fprop", M, K, N, sw)
    ctx = nv.LinearContext(M, K, N, "cuda")
    y = nv.nvfp4_linear_fwd(xc, wc, ctx, ws, signs, training=True, bf16_fprop=True, **sw)
    dx, dw = nv.nvfp4_linear_bwd(dyc, ctx, ws, signs, W.SR_SEED, **sw)
    # the same step with the NVFP4 forward: the backward must not change
    ctx0 = nv.LinearContext(M, K, N, "cuda")
    nv.nvfp4_linear_fwd(xc, wc, ctx0, ws, signs, training=True, **sw)
    dx0, dw0 = nv.nvfp4_linear_bwd(dyc, ctx0, ws, signs, W.SR_SEED, **sw)
    torch.cuda.synchronize()
    assert nv.nvfp4_device_status(ws) == nv.OK
    rec = O.Recipe(rht_signs=signs, sr_seed=W.SR_SEED, weights_2d=two_d, bf16_fprop=True)
    ops = O.linear_operands(np32(x), np32(w), np32(dy), rec)
    for name in ("wqt", "xqt", "dyq", "dyqt"):
        assert_q_equal(getattr(ctx, name), ops[name], f"{name} bf16_fprop {sw}")
    C, S = O.bf16_gemm(np32(x), np32(w))
    assert_gemm_close(y.float().cpu().numpy(), C, S, True, f"Y bf16_fprop {sw}")
    assert torch.equal(dx, dx0) and torch.equal(dw, dw0)


def test_layer_bf16_fprop_inference(nv):
    """Without training the BF16 forward quantises nothing: Y only."""
    M, K, N = 320, 512, 272
    x = W.activations(M, K, seed=W.SEED_X + 44)
    w = W.weights(N, K, seed=W.SEED_W + 44)
    ws = nv.Workspace("cuda")
    nv.nvfp4_workspace_init(ws)
    ctx = nv.LinearContext(M, K, N, "cuda")
    say("layer bf16 fprop inference", M, K, N)
    y = nv.nvfp4_linear_fwd(x.cuda(), w.cuda(), ctx, ws, 0, training=False, bf16_fprop=True)
    torch.cuda.synchronize()
    C, S = O.bf16_gemm(np32(x), np32(w))
    assert_gemm_close(y.float().cpu().numpy(), C, S, True, "Y bf16 inference")
