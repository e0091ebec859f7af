"""GPU parity of the MXFP4 comparator (nvfp4_mx_quantize, and nvfp4_gemm on
NVFP4_SCALE_MX32 operands) against the oracle: codes and E8M0 scales bit-exact,
GEMM within 1e-4 * sum|a b| (exact products, FP32 accumulation)."""
import numpy as np
import pytest
import torch

import oracle as O
from tests.gpu_util import assert_gemm_close, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import bit_quantized_numerics_amd as nv
    return nv


def _rand(rows, cols, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, cols, generator=g) * scale
    m = torch.rand(rows, cols, generator=g) < 0.01
    x[m] *= 30.0
    return x


def _check_q(q, ref, what):
    torch.cuda.synchronize()
    codes = q.codes_2d().cpu().numpy()
    scales = q.scales_2d().cpu().numpy()
    bad = np.argwhere(codes != ref.codes)
    assert bad.size == 0, f"{what}: {len(bad)} code bytes differ, first {bad[:3].tolist()}"
    bad = np.argwhere(scales != ref.scales)
    assert bad.size == 0, f"{what}: {len(bad)} scales differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("rows,cols", [(64, 256), (200, 512), (1024, 2048), (7, 96)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize(nv, rows, cols, dtype):
    x = _rand(rows, cols, rows * 7 + cols).to(dtype)
    say("mx quantize", rows, cols, dtype)
    q = nv.nvfp4_mx_quantize(x.cuda())
    _check_q(q, O.mx_quantize(x.float().numpy()), f"{rows}x{cols} {dtype}")


def test_quantize_extremes(nv):
    """Tiny, huge, subnormal, zero and NaN blocks, exact ties and saturation."""
    g = torch.Generator().manual_seed(11)
    x = torch.randn(16, 256, generator=g)
    x[0] *= 1e-30
    x[1] *= 1e30
    x[2] *= 1e-41          # fp32 subnormals
    x[3] = 0.0
    x[4, :32] = torch.tensor([7.0, 6.5, 5.0, 3.5, -0.75, 0.25, -1.25, 2.5] * 4)
    x[5, 40] = float("nan")
    x[6, 70] = float("inf")
    x[7] = (torch.randint(-16, 17, (256,), generator=g) * 0.25)
    say("mx quantize extremes")
    q = nv.nvfp4_mx_quantize(x.cuda())
    _check_q(q, O.mx_quantize(x.numpy()), "extremes")


@pytest.mark.parametrize("M,N,K", [(256, 384, 512), (200, 136, 640), (528, 400, 1024),
                                   (96, 272, 384)])
def test_gemm(nv, M, N, K):
    a, b = _rand(M, K, M + K), _rand(N, K, N * 3 + K, scale=0.02)
    say("mx gemm", M, N, K)
    qa, qb = nv.nvfp4_mx_quantize(a.cuda()), nv.nvfp4_mx_quantize(b.cuda())
    ra, rb = O.mx_quantize(a.numpy()), O.mx_quantize(b.numpy())
    C, S = O.mx_gemm(ra, rb)
    for dt in (torch.float32, torch.bfloat16):
        c = nv.nvfp4_gemm(qa, qb, dt)
        assert_gemm_close(c.float().cpu().numpy(), C, S, dt == torch.bfloat16, f"mx {M}x{N}x{K}")


@pytest.mark.slow
def test_gemm_full_fprop_sampled(nv):
    """The layer's Fprop shape in MXFP4: X [8192, 5120] x W [20480, 5120]."""
    import workloads as W
    x, w = W.activations(8192, 5120), W.weights(20480, 5120)
    say("mx gemm full fprop")
    qx, qw = nv.nvfp4_mx_quantize(x.cuda()), nv.nvfp4_mx_quantize(w.cuda())
    y = nv.nvfp4_gemm(qx, qw, torch.bfloat16)
    rx, rw = O.mx_quantize(x.float().numpy()), O.mx_quantize(w.float().numpy())
    _check_q(qx, rx, "x")
    _check_q(qw, rw, "w")
    g = np.random.default_rng(9)
    ms, ns = g.integers(0, 8192, 256), g.integers(0, 20480, 256)
    um, im = np.unique(ms, return_inverse=True)
    un, in_ = np.unique(ns, return_inverse=True)
    ah = O.mx_dequant(O.MXTensor(rx.codes[um], rx.scales[um], len(um), 5120))
    bh = O.mx_dequant(O.MXTensor(rw.codes[un], rw.scales[un], len(un), 5120))
    Cs, Ss = O.gemm_entries(ah, bh, im, in_)
    got = y[torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()].float().cpu().numpy()
    assert_gemm_close(got, Cs, Ss, True, "mx full fprop")
