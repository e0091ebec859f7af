"""GPU parity of the NVFP4 GEMM against the oracle's float64 product of the
dequantised operands: |err| <= 1e-4 * sum|a b| per element (plus the bf16
output rounding), element by element at small sizes and on sampled entries
at the layer's full sizes."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests.gpu_util import assert_gemm_close, np32, say

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


def _rand(rows, cols, seed, scale=1.0, p=0.01, mul=30.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, cols, generator=g) * scale
    m = torch.rand(rows, cols, generator=g) < p
    x[m] *= mul
    return x


def _quant_pair(nv, ws, a_np, b_np, mode_a, mode_b):
    """Quantise both operands on the GPU (already pinned bit-exact against the
    oracle by the quantiser tests) and build the oracle operands from the
    same inputs."""
    def one(x, mode):
        t = torch.from_numpy(x)
        if mode == 0:
            return nv.nvfp4_quantize(t.cuda(), ws), O.quantize(x)
        q, _ = nv.nvfp4_quantize_2d(t.cuda(), ws, want_t=False)
        return q, O.quantize_2d(x, want_t=False)[0]
    return one(a_np, mode_a), one(b_np, mode_b)


def test_tiny_config(nv, ws):
    """The tiny configuration in full: A [64, 256] 1x16 RN, B [128, 256]
    16x16 RN, C = deq(A) deq(B)^T; the same A quantised with stochastic
    rounding (Philox seed 1234, stream 0); and RHT16 of A along K (signs
    from seed 0) -- codes, scales and transformed values bit for bit."""
    from tests.gpu_util import assert_q_equal
    a, b = W.tiny_pair()
    say("gemm tiny config")
    (qa, ra), (qb, rb) = _quant_pair(nv, ws, np32(a), np32(b), 0, 1)
    assert_q_equal(qa, ra, "tiny A")
    assert_q_equal(qb, rb, "tiny B")
    C, S = O.gemm(ra, rb)
    for dt in (torch.float32, torch.bfloat16):
        c = nv.nvfp4_gemm(qa, qb, dt)
        assert_gemm_close(c.float().cpu().numpy(), C, S, dt == torch.bfloat16, f"tiny {dt}")
    q_sr = nv.nvfp4_quantize(a.cuda(), ws, round_mode=nv.SR, seed=W.SR_SEED, stream_id=0)
    assert_q_equal(q_sr, O.quantize(np32(a), sr=True, seed=W.SR_SEED, stream=0), "tiny A SR")
    signs = O.rht_signs_from_seed(W.RHT_SEED)
    y = nv.nvfp4_rht16(a.cuda(), 1, signs)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32),
                          O.rht16(np32(a), 1, signs).view(np.uint32)), "tiny A RHT16 along K"
    assert nv.nvfp4_device_status(ws) == nv.OK


# K % 128 == 0 with K >= 384 takes the LDS-slab kernel (ragged edge tiles,
# slab counts 3, 4, 5 and 8, so the four-buffer ring wraps at every phase);
# the other K take the direct-load kernel.
@pytest.mark.parametrize("M,N,K", [(80, 48, 272), (200, 136, 512), (128, 128, 64), (16, 16, 16),
                                   (256, 384, 1024), (144, 272, 48), (528, 400, 640),
                                   (96, 272, 384)])
@pytest.mark.parametrize("modes", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_shapes_and_scale_modes(nv, ws, M, N, K, modes):
    if (modes[0] == 1 and M % 16) or (modes[1] == 1 and N % 16):
        pytest.skip("16x16 needs rows % 16")
    a = np32(_rand(M, K, M + K))
    b = np32(_rand(N, K, N * 3 + K, scale=0.02))
    say("gemm", M, N, K, modes)
    (qa, ra), (qb, rb) = _quant_pair(nv, ws, a, b, *modes)
    C, S = O.gemm(ra, rb)
    c = nv.nvfp4_gemm(qa, qb, torch.float32)
    assert_gemm_close(c.cpu().numpy(), C, S, False, f"{M}x{N}x{K} {modes}")


def test_unit_scales_exact(nv):
    """All block scales 1 (E4M3 0x38) and g = 1: the product is a sum of
    multiples of 1/4 well inside fp32's exact range, so the GPU result must
    equal the exact integer product."""
    M, N, K = 96, 160, 512
    g = np.random.default_rng(0)
    a_codes = g.integers(0, 256, (M, K // 2), dtype=np.uint8)
    b_codes = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    qa, qb = nv.NVFP4Tensor(M, K, device="cuda"), nv.NVFP4Tensor(N, K, device="cuda")
    for q, codes in ((qa, a_codes), (qb, b_codes)):
        q.codes.copy_(torch.from_numpy(codes.ravel()))
        q.scales.fill_(0x38)
        q.global_scale.fill_(1.0)
    say("gemm unit scales")
    c = nv.nvfp4_gemm(qa, qb, torch.float32).cpu().numpy()
    ra = O.QTensor(a_codes, np.full((M, K // 16), 0x38, np.uint8), np.float32(1), M, K, 0)
    rb = O.QTensor(b_codes, np.full((N, K // 16), 0x38, np.uint8), np.float32(1), N, K, 0)
    C, _ = O.gemm(ra, rb)
    assert np.array_equal(c.astype(np.float64), C)


def test_large_dense_compare(nv, ws):
    M, N, K = 1024, 1536, 2048
    a = np32(_rand(M, K, 11))
    b = np32(_rand(N, K, 12, scale=0.02))
    say("gemm 1024x1536x2048")
    (qa, ra), (qb, rb) = _quant_pair(nv, ws, a, b, 0, 1)
    C, S = O.gemm(ra, rb)
    c = nv.nvfp4_gemm(qa, qb, torch.bfloat16)
    assert_gemm_close(c.float().cpu().numpy(), C, S, True, "1024x1536x2048")


def _sampled_check(nv, qa, qb, ra, rb, out_dtype, what, n_samples=384, seed=0):
    c = nv.nvfp4_gemm(qa, qb, out_dtype)
    torch.cuda.synchronize()
    M, N = ra.rows, rb.rows
    g = np.random.default_rng(seed)
    ms = np.concatenate([g.integers(0, M, n_samples), [0, M - 1, 0, M - 1]])
    ns = np.concatenate([g.integers(0, N, n_samples), [0, N - 1, N - 1, 0]])
    um, im = np.unique(ms, return_inverse=True)
    un, in_ = np.unique(ns, return_inverse=True)
    a_rows = O.dequant_rows(ra, um)
    b_rows = O.dequant_rows(rb, un)
    Cs, Ss = O.gemm_entries(a_rows, b_rows, im, in_)
    got = c[torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()].float().cpu().numpy()
    assert_gemm_close(got, Cs, Ss, out_dtype == torch.bfloat16, what)


@pytest.mark.slow
def test_full_fprop_sampled(nv, ws):
    """Fprop: X [8192, 5120] 1x16 RN x W [5120, 5120] 16x16 RN -> Y bf16."""
    x = W.activations(8192, 5120)
    w = W.weights(5120, 5120)
    say("full fprop")
    qa = nv.nvfp4_quantize(x.cuda(), ws)
    qb, _ = nv.nvfp4_quantize_2d(w.cuda(), ws, want_t=False)
    ra = O.quantize(np32(x))
    rb, _ = O.quantize_2d(np32(w), want_t=False)
    _sampled_check(nv, qa, qb, ra, rb, torch.bfloat16, "fprop")


@pytest.mark.slow
def test_full_dgrad_sampled(nv, ws):
    """Dgrad: dY [8192, 20480] 1x16 SR x W^T [5120, 20480] 16x16 -> dX bf16."""
    dy = W.gradients(8192, 20480)
    w = W.weights(20480, 5120)
    say("full dgrad")
    qa = nv.nvfp4_quantize(dy.cuda(), ws, round_mode=nv.SR, seed=W.SR_SEED)
    _, qbt = nv.nvfp4_quantize_2d(w.cuda(), ws)
    ra = O.quantize(np32(dy), sr=True, seed=W.SR_SEED)
    _, rbt = O.quantize_2d(np32(w))
    _sampled_check(nv, qa, qbt, ra, rbt, torch.bfloat16, "dgrad")


@pytest.mark.slow
def test_full_wgrad_sampled(nv, ws):
    """Wgrad: (R dY)^T [20480, 8192] SR x (R X)^T [5120, 8192] RN -> dW fp32."""
    s = O.rht_signs_from_seed(W.RHT_SEED)
    dy = W.gradients(8192, 20480)
    x = W.activations(8192, 5120)
    say("full wgrad")
    qa = nv.nvfp4_quantize(dy.cuda(), ws, round_mode=nv.SR, transpose=True, rht=True, rht_signs=s,
                           seed=W.SR_SEED, stream_id=1)
    qb = nv.nvfp4_quantize(x.cuda(), ws, transpose=True, rht=True, rht_signs=s)
    ra = O.quantize(np32(dy), transpose=True, rht=True, signs=s, sr=True, seed=W.SR_SEED, stream=1)
    rb = O.quantize(np32(x), transpose=True, rht=True, signs=s)
    _sampled_check(nv, qa, qb, ra, rb, torch.float32, "wgrad")


def test_mfma_loop_ceiling(nv):
    """The measurement helper runs and reports a plausible fp16 MFMA rate
    (above any GEMM here, below the datasheet peak)."""
    say("mfma loop ceiling")
    nv.nvfp4_peak_mfma_f16(200)
    tf = nv.nvfp4_peak_mfma_f16(2000)
    assert 500.0 < tf < 2600.0, tf
    pure = nv.nvfp4_peak_mfma_f16(2000, valu_per_mfma=0)
    assert 500.0 < pure < 2600.0, pure
    fp4 = nv.nvfp4_peak_mfma_fp4(500)
    assert 1000.0 < fp4 < 10200.0, fp4


def test_tensor_scale_rewritten_between_launches(nv, ws):
    """The GEMM reads g_A and g_B at kernel entry: re-quantising A in place
    with another tensor amax (x 64) between two launches must change the
    product accordingly (no stale value from an earlier launch)."""
    M, N, K = 512, 512, 1024
    a = np32(_rand(M, K, 41))
    b = np32(_rand(N, K, 42, scale=0.02))
    say("gemm tensor scale rewritten")
    qa = nv.nvfp4_quantize(torch.from_numpy(a).cuda(), ws)
    qb = nv.nvfp4_quantize(torch.from_numpy(b).cuda(), ws)
    rb = O.quantize(b)
    for k, scale in enumerate((1.0, 64.0, 1.0 / 8)):
        ak = a * np.float32(scale)
        nv.nvfp4_quantize(torch.from_numpy(ak).cuda(), ws, out=qa)
        ra = O.quantize(ak)
        C, S = O.gemm(ra, rb)
        c = nv.nvfp4_gemm(qa, qb, torch.float32)
        assert_gemm_close(c.cpu().numpy(), C, S, False, f"call {k} (A x {scale})")
