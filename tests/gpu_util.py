"""Helpers for the GPU parity tests: device handling, oracle conversion and
element-by-element comparison of quantised operands."""
import sys

import numpy as np
import torch

import oracle as O


def say(*a):
    """Name the case before each GPU step (flushed, so a fault still shows it)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def np32(x: torch.Tensor) -> np.ndarray:
    return x.detach().to("cpu", torch.float32).contiguous().numpy()


def assert_q_equal(gpu, ref: "O.QTensor", what=""):
    """Bit-exact equality of codes, block scales and the tensor scale."""
    torch.cuda.synchronize()
    codes = gpu.codes_2d().cpu().numpy()
    scales = gpu.scales_2d().cpu().numpy()
    g = np.float32(gpu.global_scale.cpu().item())
    assert (gpu.rows, gpu.cols) == (ref.rows, ref.cols), what
    bad = np.argwhere(codes != ref.codes)
    assert bad.size == 0, f"{what}: {len(bad)} code bytes differ, first at {bad[:3].tolist()}: " \
                          f"gpu {codes[tuple(bad[0])]:#x} ref {ref.codes[tuple(bad[0])]:#x}"
    bad = np.argwhere(scales != ref.scales)
    assert bad.size == 0, f"{what}: {len(bad)} scales differ, first at {bad[:3].tolist()}"
    assert g.tobytes() == np.float32(ref.g).tobytes(), f"{what}: g {g} vs {ref.g}"


def gemm_tolerance(S: np.ndarray, C_ref: np.ndarray, bf16_out: bool) -> np.ndarray:
    """|err| <= 1e-4 * sum|a b| (fp32 accumulation); a bf16 output adds its own
    nearest-even rounding: bf16 keeps 8 significant bits, so that error is at
    most 2^-8 of the magnitude being rounded."""
    tol = 1e-4 * S
    if bf16_out:
        tol = tol + 2.0 ** -8 * (np.abs(C_ref) + tol)
    return tol + 1e-30


def assert_gemm_close(c_gpu: np.ndarray, C_ref: np.ndarray, S: np.ndarray, bf16_out: bool, what=""):
    tol = gemm_tolerance(S, C_ref, bf16_out)
    err = np.abs(c_gpu.astype(np.float64) - C_ref)
    worst = np.unravel_index(np.argmax(err / tol), err.shape)
    assert np.all(err <= tol), (f"{what}: max err/tol {float((err / tol)[worst]):.3g} at {worst}: "
                                f"gpu {c_gpu[worst]} ref {C_ref[worst]} S {S[worst]}")
