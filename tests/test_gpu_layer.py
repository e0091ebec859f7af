"""GPU parity of the layer entry points nvfp4_linear_fwd / nvfp4_linear_bwd:
every quantised operand in the context bit-exact against the oracle's layer
composition, and the three GEMM outputs within tolerance."""
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


def _run_layer(nv, M, K, N, seed_base=0):
    x = W.activations(M, K, seed=W.SEED_X + seed_base)
    w = W.weights(N, K, seed=W.SEED_W + seed_base)
    dy = W.gradients(M, N, seed=W.SEED_DY + seed_base)
    signs = nv.nvfp4_rht_signs_from_seed(W.RHT_SEED)
    ws = nv.Workspace("cuda")
    nv.nvfp4_workspace_init(ws)
    ctx = nv.LinearContext(M, K, N, "cuda")
    say("layer", M, K, N)
    y = nv.nvfp4_linear_fwd(x.cuda(), w.cuda(), ctx, ws, signs, training=True)
    dx, dw = nv.nvfp4_linear_bwd(dy.cuda(), ctx, ws, signs, W.SR_SEED)
    torch.cuda.synchronize()
    assert nv.nvfp4_device_status(ws) == nv.OK
    ops = O.linear_operands(np32(x), np32(w), np32(dy), O.Recipe(rht_signs=signs, sr_seed=W.SR_SEED))
    for name in ("xq", "wq", "wqt", "xqt", "dyq", "dyqt"):
        assert_q_equal(getattr(ctx, name), ops[name], name)
    return ctx, ops, y, dx, dw, (x, w, dy)


# (256, 384, 512): Wgrad has K = 256 and takes the direct-load kernel, Dgrad
# the slab kernel (two launches).  (640, 272, 640): both backward GEMMs in one
# slab launch, ragged edge tiles, tile counts not multiples of 8.
# (512, 2048, 512): one launch with 16 + 16 tiles (the XCD-interleaved order).
@pytest.mark.parametrize("M,K,N", [(256, 384, 512), (640, 272, 640), (512, 2048, 512)])
def test_layer_small(nv, M, K, N):
    ctx, ops, y, dx, dw, _ = _run_layer(nv, M, K, N, seed_base=10)
    for out, (a, b), bf16, what in ((y, ("xq", "wq"), True, "Y"), (dx, ("dyq", "wqt"), True, "dX"),
                                    (dw, ("dyqt", "xqt"), False, "dW")):
        C, S = O.gemm(ops[a], ops[b])
        assert_gemm_close(out.float().cpu().numpy(), C, S, bf16, what)


@pytest.mark.parametrize("dw_dtype", [torch.float32, torch.bfloat16])
def test_layer_split_wgrad_tail(nv, dw_dtype):
    """M=512, K=2048, N=4096: the backward's one launch has 16 Dgrad tiles and
    128 Wgrad tiles, enough for the last 8 Wgrad tiles of each XCD's share to
    run as two K halves added by the combine pass.  dW (every element) is
    within the GEMM tolerance of the oracle with the split, and equals the
    unsplit result (context without scratch) exactly outside the split tiles
    and within tolerance on them."""
    M, K, N = 512, 2048, 4096
    x = W.activations(M, K, seed=W.SEED_X + 70).cuda()
    w = W.weights(N, K, seed=W.SEED_W + 70).cuda()
    dy = W.gradients(M, N, seed=W.SEED_DY + 70).cuda()
    signs = nv.nvfp4_rht_signs_from_seed(W.RHT_SEED)
    ws = nv.Workspace("cuda")
    nv.nvfp4_workspace_init(ws)
    dws = []
    for with_scratch in (True, False):
        ctx = nv.LinearContext(M, K, N, "cuda")
        if not with_scratch:
            ctx.cctx.wgrad_scratch = None
            ctx.cctx.wgrad_scratch_bytes = 0
        say("layer split", with_scratch, dw_dtype)
        nv.nvfp4_linear_fwd(x, w, ctx, ws, signs, training=True)
        _, dw = nv.nvfp4_linear_bwd(dy, ctx, ws, signs, W.SR_SEED, dw_dtype=dw_dtype)
        torch.cuda.synchronize()
        assert nv.nvfp4_device_status(ws) == nv.OK
        dws.append((ctx, dw.float().cpu().numpy()))
    (ctx, split), (_, whole) = dws
    ops = O.linear_operands(np32(x.cpu()), np32(w.cpu()), np32(dy.cpu()),
                            O.Recipe(rht_signs=signs, sr_seed=W.SR_SEED))
    assert_q_equal(ctx.dyqt, ops["dyqt"], "dyqt")
    assert_q_equal(ctx.xqt, ops["xqt"], "xqt")
    C, S = O.gemm(ops["dyqt"], ops["xqt"])
    bf16 = dw_dtype == torch.bfloat16
    assert_gemm_close(split, C, S, bf16, "dW split")
    assert_gemm_close(whole, C, S, bf16, "dW whole")
    # the split tiles (8 per XCD share, 64 of the 128) are the only ones that
    # may differ; in fp32 some of their sums do (another summation order)
    differ = split != whole
    tiles = differ.reshape(N // 256, 256, K // 256, 256).any(axis=(1, 3))
    assert tiles.sum() <= 64, int(tiles.sum())
    if not bf16:
        assert tiles.sum() > 0


def test_layer_dw_tracks_unquantised_gradient(nv):
    """The RHT cancels in dY^T X (it is orthogonal along tokens), so the NVFP4
    Wgrad stays close to the float64 dY^T X."""
    M, K, N = 512, 256, 384
    ctx, ops, y, dx, dw, (x, w, dy) = _run_layer(nv, M, K, N, seed_base=20)
    ref = np32(dy).astype(np.float64).T @ np32(x).astype(np.float64)
    rel = np.linalg.norm(dw.cpu().numpy() - ref) / np.linalg.norm(ref)
    assert rel < 0.2


@pytest.mark.slow
@pytest.mark.parametrize("M", [W.LAYER_M, 2 * W.LAYER_M])
def test_layer_full_size_sampled(nv, M):
    """The FFN up-projection 5120 -> 20480 at 8192 tokens (the benchmarked
    workload) and at 16384 tokens: every operand bit-exact, sampled outputs."""
    K, N = W.LAYER_K, W.LAYER_N
    ctx, ops, y, dx, dw, _ = _run_layer(nv, M, K, N)
    g = np.random.default_rng(5)
    for out, (a, b), bf16, what in ((y, ("xq", "wq"), True, "Y"), (dx, ("dyq", "wqt"), True, "dX"),
                                    (dw, ("dyqt", "xqt"), False, "dW")):
        ra, rb = ops[a], ops[b]
        ms = g.integers(0, ra.rows, 256)
        ns = g.integers(0, rb.rows, 256)
        um, im = np.unique(ms, return_inverse=True)
        un, in_ = np.unique(ns, return_inverse=True)
        Cs, Ss = O.gemm_entries(O.dequant_rows(ra, um), O.dequant_rows(rb, un), im, in_)
        got = out[torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()].float().cpu().numpy()
        assert_gemm_close(got, Cs, Ss, bf16, what)


def test_layer_one_buffer_context(nv):
    """A context laid out in one buffer by nvfp4_linear_ctx_init gives the same
    operands and outputs, bit for bit, as separately allocated operands."""
    M, K, N = 512, 640, 384
    x = W.activations(M, K, seed=W.SEED_X + 60).cuda()
    w = W.weights(N, K, seed=W.SEED_W + 60).cuda()
    dy = W.gradients(M, N, seed=W.SEED_DY + 60).cuda()
    signs = nv.nvfp4_rht_signs_from_seed(W.RHT_SEED)
    ws = nv.Workspace("cuda")
    nv.nvfp4_workspace_init(ws)
    outs = []
    for ctx in (nv.LinearContext(M, K, N, "cuda"), nv.LinearContext.from_buffer(M, K, N, "cuda")):
        say("layer ctx", type(ctx).__name__, M, K, N)
        y = nv.nvfp4_linear_fwd(x, w, ctx, ws, signs, training=True)
        dx, dw = nv.nvfp4_linear_bwd(dy, ctx, ws, signs, W.SR_SEED)
        torch.cuda.synchronize()
        outs.append((ctx, y, dx, dw))
    (c0, *r0), (c1, *r1) = outs
    for a, b in zip(r0, r1):
        assert torch.equal(a, b)
    for name in ("xq", "wq", "wqt", "xqt", "dyq", "dyqt"):
        q0, q1 = getattr(c0, name), getattr(c1, name)
        assert torch.equal(q0.codes_2d(), q1.codes_2d()), name
        assert torch.equal(q0.scales_2d(), q1.scales_2d()), name
        assert torch.equal(q0.global_scale, q1.global_scale), name
