"""GPU parity at the size limits the C ABI states.

- Quantiser: the largest leading dimension it accepts for bf16 rows
  (256 * ld * 2 bytes just below 2^31), row copy RN and SR and the RHT
  column copy, bit-exact against the oracle.
- NVFP4 GEMM: an operand whose codes end just below 2^31 bytes (the last
  shape the LDS-slab kernel takes with 32-bit buffer offsets) and one just
  above it (the 64-bit-addressed direct kernel), on sampled entries against
  the oracle's one-at-a-time dot products.  Codes and scales are drawn
  directly (seeded) rather than quantised, which keeps the inputs to ~2 GB.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests.gpu_util import assert_gemm_close, assert_q_equal, np32, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def nv():
    import bit_quantized_numerics_amd as nv
    return nv


@pytest.fixture(scope="module")
def ws(nv):
    w = nv.Workspace("cuda")
    nv.nvfp4_workspace_init(w)
    return w


def test_quantize_largest_leading_dim(nv, ws):
    rows, cols = 32, (1 << 22) - 16          # 256 * cols * 2 = 2^31 - 8192
    x = W.activations(rows, cols, seed=W.SEED_X + 50)
    s = O.rht_signs_from_seed(W.RHT_SEED)
    xc = x.cuda()
    say("quantize largest ld", rows, cols)
    q = nv.nvfp4_quantize(xc, ws)
    assert_q_equal(q, O.quantize(np32(x)), "row RN")
    q = nv.nvfp4_quantize(xc, ws, round_mode=nv.SR, seed=W.SR_SEED)
    assert_q_equal(q, O.quantize(np32(x), sr=True, seed=W.SR_SEED), "row SR")
    q = nv.nvfp4_quantize(xc, ws, transpose=True, rht=True, rht_signs=s)
    assert_q_equal(q, O.quantize(np32(x), transpose=True, rht=True, signs=s), "column RHT")
    assert nv.nvfp4_device_status(ws) == nv.OK


def _random_operand(nv, rows, K, gen, mode):
    q = nv.NVFP4Tensor(rows, K, mode, device="cuda")
    q.codes.copy_(torch.randint(0, 256, (q.codes.numel(),), generator=gen, device="cuda",
                                dtype=torch.uint8))
    # E4M3 codes 0x30 .. 0x3F: block scales 0.5 .. 1.875; E8M0 codes
    # 120 .. 134: 2^-7 .. 2^7
    lo, hi = (0x30, 0x40) if mode == nv.SCALE_1X16 else (120, 135)
    q.scales.copy_(torch.randint(lo, hi, (q.scales.numel(),), generator=gen, device="cuda",
                                 dtype=torch.uint8))
    q.global_scale.fill_(1.0)
    return q


def _rows_oracle(nv, q, rows):
    idx = torch.from_numpy(rows).cuda()
    codes = q.codes_2d()[idx].cpu().numpy()
    scales = q.scales_2d()[idx].cpu().numpy()
    if q.scale_mode == nv.SCALE_MX32:
        return O.mx_dequant(O.MXTensor(codes, scales, rows.size, q.cols))
    return O.dequant(O.QTensor(codes, scales, np.float32(1.0), rows.size, q.cols, 0))


def _samples(M, N, seed):
    g = np.random.default_rng(seed)
    ms = np.concatenate([g.integers(0, M, 48), [0, M - 1, M - 1, 0, M // 2]])
    ns = np.concatenate([g.integers(0, N, 48), [0, N - 1, 0, N - 1, N // 2]])
    return ms, ns


# A [M, 1024]: M * 512 code bytes is 2^31 - 2^20 (the last shapes the
# LDS-slab kernels take with 32-bit buffer offsets) or exactly 2^31 (NVFP4
# falls back to the 64-bit-addressed direct kernel).  B [256, 1024].
@pytest.mark.parametrize("M,path", [((1 << 22) - 2048, "slab"), (1 << 22, "direct"),
                                    ((1 << 22) - 2048, "mx")])
def test_gemm_operand_offset_limit(nv, M, path):
    N, K = 256, 1024
    gen = torch.Generator(device="cuda")
    gen.manual_seed(51)
    mode = nv.SCALE_MX32 if path == "mx" else nv.SCALE_1X16
    say("gemm offset limit", M, N, K, path)
    qa = _random_operand(nv, M, K, gen, mode)
    qb = _random_operand(nv, N, K, gen, mode)
    c = nv.nvfp4_gemm(qa, qb, torch.float32)
    torch.cuda.synchronize()
    ms, ns = _samples(M, N, 52)
    um, im = np.unique(ms, return_inverse=True)
    un, in_ = np.unique(ns, return_inverse=True)
    Cs, Ss = O.gemm_entries(_rows_oracle(nv, qa, um), _rows_oracle(nv, qb, un), im, in_)
    got = c[torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()].cpu().numpy()
    assert_gemm_close(got, Cs, Ss, False, f"offset limit {path}")


def test_bf16_gemm_operand_offset_limit(nv):
    """A bf16 [2^20 - 256, 1024]: its rows rounded up to 256, times 2 KiB,
    is 2^31 - 2^19, the largest nvfp4_bf16_gemm accepts at this K."""
    M, N, K = (1 << 20) - 256, 256, 1024
    gen = torch.Generator(device="cuda")
    gen.manual_seed(53)
    say("bf16 gemm offset limit", M, N, K)
    a = torch.randn(M, K, generator=gen, device="cuda").to(torch.bfloat16)
    b = torch.randn(N, K, generator=gen, device="cuda").to(torch.bfloat16)
    c = nv.nvfp4_bf16_gemm(a, b, torch.float32)
    torch.cuda.synchronize()
    ms, ns = _samples(M, N, 54)
    um, im = np.unique(ms, return_inverse=True)
    un, in_ = np.unique(ns, return_inverse=True)
    a_rows = O.bf16_values(np32(a[torch.from_numpy(um).cuda()]))
    b_rows = O.bf16_values(np32(b[torch.from_numpy(un).cuda()]))
    Cs, Ss = O.gemm_entries(a_rows, b_rows, im, in_)
    got = c[torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()].cpu().numpy()
    assert_gemm_close(got, Cs, Ss, False, "bf16 offset limit")
