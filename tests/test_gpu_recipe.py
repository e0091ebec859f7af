"""GPU parity of the recipe switches and of nvfp4_dequantize.

- Each ablation of the pages' recipe [Captions Fig. 4, 10, 11, 14] through
  nvfp4_linear_fwd/bwd: every quantised operand bit-exact against the
  oracle's layer composition with the same switches, GEMMs within tolerance.
- nvfp4_dequantize bit-exact against the oracle's float64 decode rounded to
  fp32 (e2m1 * d_b is exact, so both round the same exact product once).
- The weight-consistency measurement [Review s2; Captions Fig. 14]: with
  16x16 scales the Dgrad copy of W decodes to exactly the Fprop copy
  transposed; with 1x16 scales along each copy's own rows it does not.
"""
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


SWITCHES = [dict(no_2d_weights=True), dict(no_rht=True), dict(no_sr=True),
            dict(no_2d_weights=True, no_rht=True, no_sr=True)]


@pytest.mark.parametrize("sw", SWITCHES, ids=lambda d: "+".join(k for k in d))
@pytest.mark.parametrize("M,K,N", [(256, 384, 512), (512, 2048, 512)])
def test_layer_ablations(nv, sw, M, K, N):
    x = W.activations(M, K, seed=W.SEED_X + 30)
    w = W.weights(N, K, seed=W.SEED_W + 30)
    dy = W.gradients(M, N, seed=W.SEED_DY + 30)
    signs = nv.nvfp4_rht_signs_from_seed(W.RHT_SEED)
    ws = nv.Workspace("cuda")
    nv.nvfp4_workspace_init(ws)
    ctx = nv.LinearContext(M, K, N, "cuda")
    say("layer ablation", sw, M, K, N)
    y = nv.nvfp4_linear_fwd(x.cuda(), w.cuda(), ctx, ws, signs, training=True, **sw)
    dx, dw = nv.nvfp4_linear_bwd(dy.cuda(), ctx, ws, signs, W.SR_SEED, **sw)
    torch.cuda.synchronize()
    assert nv.nvfp4_device_status(ws) == nv.OK
    rec = O.Recipe(rht_signs=signs, sr_seed=W.SR_SEED, weights_2d=not sw.get("no_2d_weights"),
                   rht=not sw.get("no_rht"), sr=not sw.get("no_sr"))
    ops = O.linear_operands(np32(x), np32(w), np32(dy), rec)
    for name in ("xq", "wq", "wqt", "xqt", "dyq", "dyqt"):
        assert_q_equal(getattr(ctx, name), ops[name], f"{name} {sw}")
    for out, (a, b), bf16, what in ((y, ("xq", "wq"), True, "Y"), (dx, ("dyq", "wqt"), True, "dX"),
                                    (dw, ("dyqt", "xqt"), False, "dW")):
        C, S = O.gemm(ops[a], ops[b])
        assert_gemm_close(out.float().cpu().numpy(), C, S, bf16, f"{what} {sw}")


@pytest.mark.parametrize("mode", ["1x16", "16x16", "mx32"])
def test_dequantize(nv, mode):
    g = torch.Generator().manual_seed(21)
    x = torch.randn(96, 256, generator=g) * 3.0
    x[5] *= 1e-6
    x[7, 3] = 400.0
    say("dequantize", mode)
    if mode == "1x16":
        ws = nv.Workspace("cuda"); nv.nvfp4_workspace_init(ws)
        q = nv.nvfp4_quantize(x.cuda(), ws)
        ref = O.dequant(O.quantize(x.numpy()))
    elif mode == "16x16":
        ws = nv.Workspace("cuda"); nv.nvfp4_workspace_init(ws)
        q, _ = nv.nvfp4_quantize_2d(x.cuda(), ws, want_t=False)
        ref = O.dequant(O.quantize_2d(x.numpy(), want_t=False)[0])
    else:
        q = nv.nvfp4_mx_quantize(x.cuda())
        ref = O.mx_dequant(O.mx_quantize(x.numpy()))
    got = nv.nvfp4_dequantize(q).cpu().numpy()
    want = ref.astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
        f"{np.count_nonzero(got != want)} values differ"


def test_weight_consistency(nv):
    """w_fprop vs w_bprop: identical under 16x16 scales, different under 1x16."""
    N, K = 512, 768
    w = W.weights(N, K, seed=77).cuda()
    ws = nv.Workspace("cuda"); nv.nvfp4_workspace_init(ws)
    say("weight consistency")
    q2, q2t = nv.nvfp4_quantize_2d(w, ws)
    a, b = nv.nvfp4_dequantize(q2), nv.nvfp4_dequantize(q2t)
    assert torch.equal(a, b.t())
    q1 = nv.nvfp4_quantize(w, ws)
    q1t = nv.nvfp4_quantize(w, ws, transpose=True)
    a1, b1 = nv.nvfp4_dequantize(q1), nv.nvfp4_dequantize(q1t)
    rel = (torch.linalg.norm(a1 - b1.t()) / torch.linalg.norm(a1)).item()
    assert rel > 1e-3   # the copies disagree
    # and the oracle sees the same disagreement
    ref = O.dequant(O.quantize(np32(w)))
    ref_t = O.dequant(O.quantize(np32(w), transpose=True))
    rel_ref = np.linalg.norm(ref - ref_t.T) / np.linalg.norm(ref)
    assert rel == pytest.approx(rel_ref, rel=1e-5)


@pytest.mark.parametrize("two_d", [True, False], ids=["2d", "1x16"])
def test_inference_forward(nv, two_d):
    """training = False: X and W quantised for Fprop only (no backward copies),
    Y against the oracle's product of the same operands."""
    M, K, N = 320, 512, 272
    x = W.activations(M, K, seed=W.SEED_X + 70)
    w = W.weights(N, K, seed=W.SEED_W + 70)
    ws = nv.Workspace("cuda")
    nv.nvfp4_workspace_init(ws)
    ctx = nv.LinearContext(M, K, N, "cuda")
    say("inference forward", M, K, N, two_d)
    y = nv.nvfp4_linear_fwd(x.cuda(), w.cuda(), ctx, ws, 0, training=False,
                            no_2d_weights=not two_d)
    torch.cuda.synchronize()
    assert nv.nvfp4_device_status(ws) == nv.OK
    ops = O.linear_operands(np32(x), np32(w), None, O.Recipe(rht_signs=0, weights_2d=two_d))
    assert_q_equal(ctx.xq, ops["xq"], "xq")
    assert_q_equal(ctx.wq, ops["wq"], "wq")
    C, S = O.gemm(ops["xq"], ops["wq"])
    assert_gemm_close(y.float().cpu().numpy(), C, S, True, "Y inference")
