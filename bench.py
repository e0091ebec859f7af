"""Benchmark: NVFP4 linear layer forward + backward on one MI355X.

One step = the whole hot path of one training step of the layer
Y = X W^T (X [8192, 5120], W [20480, 5120], dY [8192, 20480], bf16 inputs
resident in HBM): quantise X (row copy + RHT'd column copy), W (16x16 scales +
transposed copy) and dY (stochastic row copy + RHT'd stochastic column copy),
then the Fprop, Dgrad and Wgrad GEMMs.  The timed step calls the C ABI entry
points nvfp4_linear_fwd and nvfp4_linear_bwd.

value = 3 * 2 * M * N * K / step time  (TFLOP/s, whole job, one GPU).
A second timed pass issues the same kernels through the per-operation entry
points with HIP events between them on the launch stream, giving the
per-phase times behind `quantize_GBps` and the GEMM roofline.  A third times
each step alone between HIP events, with a 512 MB scratch write before it so
that nothing is left in the memory-side cache, and reports the median of 20
(`step_ms_event_median_flushed`).  `measured_ceiling` holds what the card
sustains on a plain 1 GiB device copy and on MFMA-only loops.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NVFP4 linear fwd+bwd TFLOP/s + quantize GB/s (8192 tok, 5120→20480)"
M, K, N = 8192, 5120, 20480
PEAK_F16_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBPS = 8000.0
PEAK_FP4_TFLOPS = 10100.0  # MI355X dense fp4 MFMA (the MXFP4 comparator's dtype)

# Algorithmic bytes of the quantisers, per source element (bf16 input):
# read 2 B; each copy writes 0.5 B of codes + 1/16 B of 1x16 scales, or
# 1/256 B of 16x16 scales.
BYTES_ROWCOL = 2.0 + 2 * (0.5 + 1.0 / 16)
BYTES_2D = 2.0 + 2 * (0.5 + 1.0 / 256)
# As run: the tensor amax is a pass of its own before the emit pass, so the
# source is read twice.
BYTES_ROWCOL_RUN = BYTES_ROWCOL + 2.0
BYTES_2D_RUN = BYTES_2D + 2.0

# HBM traffic of the GEMM kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE
# (KiB per dispatch; FETCH_SIZE x 2 and WRITE_SIZE x 1, the factors a plain
# 1 GiB device copy reads back), averaged over the single Fprop, Dgrad and
# Wgrad launches: 999.4, 790.3 and 1243.9 MB.  Valid only for the kernel
# source it was measured on (profiles/hbm_traffic_gemm_quantize_*.md).
GEMM_TRAFFIC = {"source_sha1": "ed02f68775c7e418de31a51cf6e8325fdab15199",
                "bytes_per_launch": 1011.2e6}


def _gemm_source_sha1() -> str:
    with open(os.path.join(ROOT, "bit_quantized_numerics_amd", "csrc", "gemm.hip"), "rb") as f:
        return hashlib.sha1(f.read()).hexdigest()


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=8192)
    p.add_argument("--copy-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB (5 times) and exit: the "
                        "known-size reference for scaling HBM byte counters")
    return p.parse_args()


def copy_reference(mib: int) -> None:
    """Five launches of torch's device-to-device copy over `mib` MiB: each
    reads and writes exactly mib MiB, so a profiler's per-dispatch byte
    counters over these launches give the counters' scale."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_mib": mib, "launches": 5, "bytes_read_per_launch": n * 4,
                      "bytes_written_per_launch": n * 4}), flush=True)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(sample_tokens: int):
    """The oracle, as it stands, on a bounded sample of the same step: the
    layer with `sample_tokens` tokens (W stays full size): the six
    quantisations, then the three products C = deq(A) deq(B)^T (float64)."""
    import oracle as O
    import workloads as W
    Ms = sample_tokens
    x = W.activations(Ms, K).float().numpy()
    w = W.weights(N, K).float().numpy()
    dy = W.gradients(Ms, N).float().numpy()
    signs = O.rht_signs_from_seed(W.RHT_SEED)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t0 = time.perf_counter()
    ops = O.linear_operands(x, w, dy, O.Recipe(rht_signs=signs, sr_seed=W.SR_SEED))
    t1 = time.perf_counter()
    for a, b in (("xq", "wq"), ("dyq", "wqt"), ("dyqt", "xqt")):
        O.gemm_c(ops[a], ops[b])
    t2 = time.perf_counter()
    flops = 3 * 2.0 * Ms * N * K
    qbytes = BYTES_ROWCOL * (Ms * K + Ms * N) + BYTES_2D * N * K
    return {
        "value": flops / (t2 - t0) / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "cpu_model": _cpu_model(), "cpus_online": os.cpu_count(),
        "sample": f"one layer step at {Ms} tokens (K={K}, N={N}, W full size): all six "
                  f"quantisations + three float64 products C = deq(A) deq(B)^T; {t2 - t0:.2f} s",
        "quantize_GBps": qbytes / (t1 - t0) / 1e9,
    }


def rht_sizes(nv, x, ws, reps: int):
    """The Wgrad copy of X, (R_d X)^T quantised along tokens, at the layer's
    shape: d = 16 (the recipe) and d = 4 fused into the quantiser, d = 128 as
    nvfp4_rht followed by nvfp4_quantize of the transpose (HIP events)."""
    import torch
    signs16 = nv.nvfp4_rht_signs_from_seed(0)
    signs = nv.nvfp4_rht_signs128_from_seed(0)
    y = torch.empty(M, K, dtype=torch.float32, device=x.device)
    q = nv.nvfp4_quantize(x, ws, transpose=True, rht=True, rht_signs=signs16)

    def d16():
        nv.nvfp4_quantize(x, ws, q, transpose=True, rht=True, rht_signs=signs16)

    def d4():
        nv.nvfp4_quantize(x, ws, q, transpose=True, rht=True, rht_d=4, rht_signs=signs16)

    def dd(d):
        def f():
            nv.nvfp4_rht(x, 0, d, signs, y)
            nv.nvfp4_quantize(y, ws, q, transpose=True)
        return f

    out = {"workload": f"(R_d X)^T, X [{M}, {K}] bf16, quantised along tokens"}
    stream = torch.cuda.current_stream()
    for name, f in (("d16_fused_ms", d16), ("d4_fused_ms", d4), ("d128_ms", dd(128))):
        f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        out[name] = round(e0.elapsed_time(e1) / reps, 4)
    return out


def weight_consistency(nv, w, ws):
    """w_fprop vs w_bprop [Review s2; Captions Fig. 14]: relative Frobenius
    difference between the decoded Fprop copy of W and the decoded Dgrad copy
    (transposed back), with 16x16 scales (the recipe) and with 1x16 scales
    along each copy's own rows (the ablation)."""
    import torch

    def rel(a, b):
        da, db = nv.nvfp4_dequantize(a), nv.nvfp4_dequantize(b).t()
        return float((torch.linalg.norm(da - db) / torch.linalg.norm(da)).item())

    q2, q2t = nv.nvfp4_quantize_2d(w, ws)
    r2 = rel(q2, q2t)
    q1, q1t = nv.nvfp4_quantize(w, ws), nv.nvfp4_quantize(w, ws, transpose=True)
    r1 = rel(q1, q1t)
    return {"workload": f"W [{N}, {K}], decoded Fprop copy vs transposed decoded Dgrad copy",
            "rel_diff_16x16": r2, "rel_diff_1x16": r1}


def mxfp4_comparator(nv, x, w, reps: int):
    """The pages' comparator format on the same Fprop shape: MXFP4 quantisation
    of X and W (32-element blocks, E8M0 scales) and the GEMM on gfx950's
    scaled FP4 MFMA (exact products, FP32 accumulation), timed with HIP
    events on the launch stream."""
    import torch
    qx = nv.nvfp4_mx_quantize(x)
    qw = nv.nvfp4_mx_quantize(w)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=x.device)
    for _ in range(2):
        nv.nvfp4_mx_quantize(x, qx)
        nv.nvfp4_mx_quantize(w, qw)
        nv.nvfp4_gemm(qx, qw, c=y)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    tq = tg = 0.0
    for _ in range(reps):
        ev[0].record(stream)
        nv.nvfp4_mx_quantize(x, qx)
        nv.nvfp4_mx_quantize(w, qw)
        ev[1].record(stream)
        nv.nvfp4_gemm(qx, qw, c=y)
        ev[2].record(stream)
        torch.cuda.synchronize()
        tq += ev[0].elapsed_time(ev[1])
        tg += ev[1].elapsed_time(ev[2])
    tq, tg = tq / reps, tg / reps
    tflops = 2.0 * M * N * K / (tg * 1e-3) / 1e12
    return {"workload": f"Fprop {M}x{K} by {N}x{K} in MXFP4, bf16 out",
            "quantize_x_w_ms": round(tq, 4), "gemm_ms": round(tg, 4),
            "gemm_TFLOPs": round(tflops, 1), "peak_fp4_TFLOPs": PEAK_FP4_TFLOPS,
            "frac": round(tflops / PEAK_FP4_TFLOPS, 4)}


def bf16_fprop(nv, x, w, ctx, ws, signs, reps: int):
    """The precision switch's forward [Review "Core strengths" item 9;
    Captions Fig. 7] on the Fprop shape: the plain BF16 GEMM alone, and the training forward with
    bf16_fprop (backward copies of X and W, then the BF16 GEMM) next to the
    NVFP4 training forward, timed with HIP events on the launch stream."""
    import torch
    y = torch.empty(M, N, dtype=torch.bfloat16, device=x.device)
    runs = [lambda: nv.nvfp4_bf16_gemm(x, w, c=y),
            lambda: nv.nvfp4_linear_fwd(x, w, ctx, ws, signs, training=True, y=y, bf16_fprop=True),
            lambda: nv.nvfp4_linear_fwd(x, w, ctx, ws, signs, training=True, y=y)]
    for _ in range(2):
        for f in runs:
            f()
    stream = torch.cuda.current_stream()
    tot = [0.0] * len(runs)
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(runs) + 1)]
        ev[0].record(stream)
        for i, f in enumerate(runs):
            f()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        for i in range(len(runs)):
            tot[i] += ev[i].elapsed_time(ev[i + 1])
    tg, tf, tn = (t / reps for t in tot)
    tflops = 2.0 * M * N * K / (tg * 1e-3) / 1e12
    return {"workload": f"Fprop {M}x{K} by {N}x{K} in BF16 (no quantisation), bf16 out",
            "gemm_ms": round(tg, 4), "gemm_TFLOPs": round(tflops, 1),
            "peak_bf16_TFLOPs": PEAK_F16_TFLOPS, "frac": round(tflops / PEAK_F16_TFLOPS, 4),
            "layer_fwd_bf16_fprop_ms": round(tf, 4), "layer_fwd_nvfp4_ms": round(tn, 4)}


def hbm_copy_rate(reps: int) -> float:
    """GB/s of torch's device-to-device copy over 1 GiB (read 1 GiB + write
    1 GiB per launch), median of `reps` launches timed with HIP events."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    stream = torch.cuda.current_stream()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts.sort()
    return 2.0 * n * 4 / (ts[len(ts) // 2] * 1e-3) / 1e9


def layer_at(nv, W, m: int, signs: int, reps: int):
    """The whole layer step (all quantisations and the three GEMMs, one stream)
    at m tokens: X [m, K], W [N, K], dY [m, N] from the same generators."""
    import torch
    dev = "cuda:0"
    x = W.activations(m, K).to(dev)
    w = W.weights(N, K).to(dev)
    dy = W.gradients(m, N).to(dev)
    ws = nv.Workspace(dev)
    nv.nvfp4_workspace_init(ws)
    ctx = nv.LinearContext(m, K, N, dev)
    y = torch.empty(m, N, dtype=torch.bfloat16, device=dev)
    dx = torch.empty(m, K, dtype=torch.bfloat16, device=dev)
    dw = torch.empty(N, K, dtype=torch.float32, device=dev)

    def step():
        nv.nvfp4_linear_fwd(x, w, ctx, ws, signs, training=True, y=y)
        nv.nvfp4_linear_bwd(dy, ctx, ws, signs, W.SR_SEED, dx=dx, dw=dw)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / reps * 1e3
    assert nv.nvfp4_device_status(ws) == nv.OK
    return {"workload": f"NVFP4 linear layer fwd+bwd, {m} tokens, {K}->{N}", "steps": reps,
            "ms_per_step": round(ms, 4), "TFLOPs": round(3 * 2.0 * m * N * K / (ms * 1e-3) / 1e12, 1)}


def main():
    args = parse()
    if args.copy_mib:
        copy_reference(args.copy_mib)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_quantized_numerics_amd as nv
    import workloads as W

    dev = "cuda:0"
    torch.cuda.set_device(0)
    x = W.activations(M, K).to(dev)
    w = W.weights(N, K).to(dev)
    dy = W.gradients(M, N).to(dev)
    signs = nv.nvfp4_rht_signs_from_seed(W.RHT_SEED)
    ws = nv.Workspace(dev)
    nv.nvfp4_workspace_init(ws)
    ctx = nv.LinearContext(M, K, N, dev)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    dx = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    dw = torch.empty(N, K, dtype=torch.float32, device=dev)

    def step():
        nv.nvfp4_linear_fwd(x, w, ctx, ws, signs, training=True, y=y)
        nv.nvfp4_linear_bwd(dy, ctx, ws, signs, W.SR_SEED, dx=dx, dw=dw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert nv.nvfp4_device_status(ws) == nv.OK
    ms_per_step = (t1 - t0) / args.steps * 1e3
    flops = 3 * 2.0 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12

    # ---- per-phase breakdown: the same kernels through the per-op entry points
    stream = torch.cuda.current_stream()
    names = ["quant_x", "quant_w", "gemm_fprop", "quant_dy", "gemm_dgrad", "gemm_wgrad"]

    def phases():
        yield lambda: nv.nvfp4_quantize_rowcol(x, ws, ctx.xq, ctx.xqt, rht=True, rht_signs=signs)
        yield lambda: nv.nvfp4_quantize_2d(w, ws, ctx.wq, ctx.wqt)
        yield lambda: nv.nvfp4_gemm(ctx.xq, ctx.wq, c=y)
        yield lambda: nv.nvfp4_quantize_rowcol(dy, ws, ctx.dyq, ctx.dyqt, round_row=nv.SR,
                                               round_col=nv.SR, rht=True, rht_signs=signs,
                                               seed=W.SR_SEED)
        yield lambda: nv.nvfp4_gemm(ctx.dyq, ctx.wqt, c=dx)
        yield lambda: nv.nvfp4_gemm(ctx.dyqt, ctx.xqt, c=dw)

    for _ in range(2):
        for f in phases():
            f()
    torch.cuda.synchronize()
    reps = max(3, args.steps // 2)
    tot = {n: 0.0 for n in names}
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        ev[0].record(stream)
        for i, f in enumerate(phases()):
            f()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        for i, n in enumerate(names):
            tot[n] += ev[i].elapsed_time(ev[i + 1])
    ph = {n: tot[n] / reps for n in names}  # ms
    gemm_ms = (ph["gemm_fprop"] + ph["gemm_dgrad"] + ph["gemm_wgrad"]) / 3
    quant_ms = ph["quant_x"] + ph["quant_w"] + ph["quant_dy"]
    qbytes = BYTES_ROWCOL * (M * K + M * N) + BYTES_2D * N * K
    qbytes_run = BYTES_ROWCOL_RUN * (M * K + M * N) + BYTES_2D_RUN * N * K
    gemm_flops = 2.0 * M * N * K
    achieved = gemm_flops / (gemm_ms * 1e-3) / 1e12
    traffic = None
    if GEMM_TRAFFIC["source_sha1"] == _gemm_source_sha1():
        traffic = GEMM_TRAFFIC["bytes_per_launch"]

    # the same step timed as one HIP-event interval per step on the launch
    # stream, a 512 MB scratch write between steps so that no operand is
    # left in the 256 MB memory-side cache, median of 20
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    ev_t = []
    for i in range(20):
        flush.fill_(i & 0x7F)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        ev_t.append(e0.elapsed_time(e1))
    del flush
    ev_t.sort()
    step_median_ms = 0.5 * (ev_t[9] + ev_t[10])
    copy_gbps = hbm_copy_rate(5)

    def qphase(name, elems, b_alg, b_run):
        t = ph[name] * 1e-3
        alg = elems * b_alg / t / 1e9
        return {"elements": elems, "ms": round(ph[name], 4), "GBps": round(alg, 1),
                "frac_of_hbm_peak": round(alg / PEAK_HBM_GBPS, 4),
                "frac_of_measured_copy": round(alg / copy_gbps, 4),
                "GBps_two_pass_bytes": round(elems * b_run / t / 1e9, 1),
                "two_pass_frac_of_hbm_peak": round(elems * b_run / t / 1e9 / PEAK_HBM_GBPS, 4)}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "NVFP4 linear layer fwd+bwd (Fprop+Dgrad+Wgrad, all quantisations), "
                               "8192 tokens, 5120->20480",
                   "M": M, "K": K, "N": N, "input_dtype": "bf16", "y_dx_dtype": "bf16",
                   "dw_dtype": "f32", "recipe": "2D W scales, RHT16 on Wgrad inputs, SR on dY"},
        "step_ms_event_median_flushed": round(step_median_ms, 4),
        "TFLOPs_event_median_flushed": round(3 * gemm_flops / (step_median_ms * 1e-3) / 1e12, 2),
        "quantize_GBps": round(qbytes / (quant_ms * 1e-3) / 1e9, 1),
        "quantize_frac_of_hbm_peak": round(qbytes / (quant_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "quantize_frac_of_measured_copy": round(qbytes / (quant_ms * 1e-3) / 1e9 / copy_gbps, 4),
        "quantize_two_pass_GBps": round(qbytes_run / (quant_ms * 1e-3) / 1e9, 1),
        "quantize_two_pass_frac_of_hbm_peak": round(qbytes_run / (quant_ms * 1e-3) / 1e9
                                                    / PEAK_HBM_GBPS, 4),
        "quantize_phases": {
            "x_row_and_rht_col": qphase("quant_x", M * K, BYTES_ROWCOL, BYTES_ROWCOL_RUN),
            "w_16x16_and_transposed": qphase("quant_w", N * K, BYTES_2D, BYTES_2D_RUN),
            "dy_sr_row_and_sr_rht_col": qphase("quant_dy", M * N, BYTES_ROWCOL, BYTES_ROWCOL_RUN)},
        "phase_ms": {n: round(v, 4) for n, v in ph.items()},
        "roofline": {"bound": "mfma", "kernel": "nvfp4 gemm (f16 MFMA, fp32 acc), avg of 3 launches",
                     "achieved": round(achieved, 2), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_F16_TFLOPS, 4), "traffic": traffic},
    }
    out["mxfp4_comparator"] = mxfp4_comparator(nv, x, w, max(3, args.steps // 2))
    out["weight_consistency"] = weight_consistency(nv, w, ws)
    out["rht_sizes"] = rht_sizes(nv, x, ws, max(3, args.steps // 2))
    out["bf16_fprop"] = bf16_fprop(nv, x, w, ctx, ws, signs, max(3, args.steps // 2))
    # the compute ceiling the card holds under a sustained fp16 MFMA load (no
    # memory traffic), next to the datasheet peak used in `roofline`
    nv.nvfp4_peak_mfma_f16(1000)
    mfma_pure = nv.nvfp4_peak_mfma_f16(5000, valu_per_mfma=0)
    mfma_pure_6bit = nv.nvfp4_peak_mfma_f16(5000, toggle_mask=0x87E087E0, valu_per_mfma=0)
    mfma_loop = nv.nvfp4_peak_mfma_f16(5000)
    mfma_6bit = nv.nvfp4_peak_mfma_f16(5000, toggle_mask=0x87E087E0)
    mfma_const = nv.nvfp4_peak_mfma_f16(5000, toggle_mask=0, valu_per_mfma=0)
    nv.nvfp4_peak_mfma_fp4(500)
    mfma_fp4 = nv.nvfp4_peak_mfma_fp4(2500)
    mx = out["mxfp4_comparator"]
    mx["frac_of_fp4_loop"] = round(mx["gemm_TFLOPs"] / mfma_fp4, 4)
    out["measured_ceiling"] = {
        "hbm_copy_GBps": round(copy_gbps, 1),
        "mfma_f16_pure_TFLOPs": round(mfma_pure, 1),
        "mfma_f16_pure_6bit_operands_TFLOPs": round(mfma_pure_6bit, 1),
        "mfma_f16_pure_constant_operands_TFLOPs": round(mfma_const, 1),
        "mfma_f16_4valu_TFLOPs": round(mfma_loop, 1),
        "mfma_f16_4valu_6bit_operands_TFLOPs": round(mfma_6bit, 1),
        "gemm_frac_of_pure": round(achieved / mfma_pure, 4),
        "gemm_frac_of_pure_6bit": round(achieved / mfma_pure_6bit, 4),
        "mfma_fp4_scaled_pure_TFLOPs": round(mfma_fp4, 1),
        "note": "hbm_copy: torch's device copy of 1 GiB (reads and writes 1 GiB), median of 5, "
                "HIP events. mfma: an fp16 32x32x16 MFMA loop with 16 accumulators per wave and "
                "one wave per SIMD, as the GEMM runs; 'pure' issues no VALU between MFMAs, "
                "'4valu' issues 4 independent VALU ops after each; operands alternate between "
                "two register sets differing in sign, one exponent bit and all mantissa bits, or "
                "in sign, that exponent bit and the top 5 mantissa bits (the bit pattern of "
                "dequantised E2M1 x E4M3 values, at most 6 significant bits), or stay constant. "
                "mfma_fp4_scaled: the MXFP4 comparator's scaled FP4 MFMA (32x32x64, E2M1 x E2M1, "
                "unit scales) in the same VALU-free loop, all code bits toggling"}
    out["layer_16384_tokens"] = layer_at(nv, W, 2 * M, signs, max(3, args.steps // 4))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
