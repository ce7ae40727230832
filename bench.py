"""Benchmark of the W4A16 hot path on one MI355X.

Step = one call of wq_gemm_w4a16 (the fused dequantize-and-multiply) on the
decode workload M=1, N=K=8192, group 128, with seeded synthetic bf16 weights
(quantized once on the GPU before timing) and fp16 activations, all resident
in HBM.  The weights are replicated into enough copies (>= 512 MB) that
consecutive steps never find them in the 256 MB last-level cache.

value = effective GB/s = algorithmic bytes (4-bit codes + fp16 scales + 4-bit
zero-points + fp16 x + fp16 y) / time per step.  The M=128 GEMM (TFLOP/s), the
quantization kernel and the CPU oracle are reported alongside in the same line.

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 20]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, AMD published
FP16_PEAK_TFLOPS = 2516.6       # MI355X dense fp16 MFMA, AMD published (256 CU x 4096 FLOP/clk x 2.4 GHz)
METRIC = "W4A16 GEMV effective HBM GB/s (% of peak) at M=1; GEMM TFLOP/s at M=128"
ROTATE_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _ensure_built():
    import w4a16_bit_matmul_amd as wq
    if not os.path.exists(wq.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()


def _device_copies(qw, copies):
    import torch
    import w4a16_bit_matmul_amd as wq
    out = [qw]
    for _ in range(copies - 1):
        out.append(wq.QuantizedWeight(qw.qpacked.clone(), qw.s.clone(), qw.zpacked.clone(), qw.N, qw.K, qw.group))
    torch.cuda.synchronize()
    return out


def _quantize_workload(wl):
    import numpy as np
    import torch
    import w4a16_bit_matmul_amd as wq
    t0 = time.time()
    W = wl.weights()
    Wd = torch.from_numpy(W.view(np.int16)).cuda().view(torch.bfloat16)
    x = wl.activations()
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.float16)
    log(f"[bench] generated {wl.name} inputs in {time.time() - t0:.1f}s")
    qw = wq.wq_quantize_groups(Wd, wl.group)["qw"]
    torch.cuda.synchronize()
    return Wd, xd, qw


def _time_calls(fn, n_calls, warmup):
    """Average GPU time per call from events on the launch stream."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n_calls):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / n_calls  # seconds per call


def bench_gemv(steps, warmup):
    import torch
    import w4a16_bit_matmul_amd as wq
    import workloads
    wl = workloads.WORKLOADS["decode_gemv"]
    Wd, xd, qw = _quantize_workload(wl)
    del Wd
    nbytes = wl.algorithmic_bytes()
    copies = max(2, math.ceil(ROTATE_BYTES / nbytes))
    qws = _device_copies(qw, copies)
    y = torch.empty((wl.M, wl.N), dtype=torch.float16, device="cuda")

    def step(i):
        wq.wq_gemm_w4a16(xd, qws[i % copies], y=y)

    # eager: one launch per step, back to back on the current stream
    torch.cuda.synchronize()
    t_eager = _time_calls(step, steps, warmup)
    # the same launches replayed from a HIP graph (removes host launch gaps)
    per_graph = copies
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(per_graph):
            step(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            step(i)
    reps = max(1, math.ceil(steps / per_graph))
    t_graph = _time_calls(lambda i: g.replay(), reps, max(1, warmup // per_graph)) / per_graph
    return wl, nbytes, copies, t_eager, t_graph, (xd, qw, y)


def bench_gemm(steps, warmup):
    import torch
    import w4a16_bit_matmul_amd as wq
    import workloads
    wl = workloads.WORKLOADS["batched_gemm"]
    Wd, xd, qw = _quantize_workload(wl)
    copies = max(2, math.ceil(ROTATE_BYTES / wl.algorithmic_bytes()))
    # dense fp16 reference point of the same shape (weights as fp16)
    Wf = Wd.to(torch.float16)
    del Wd
    qws = _device_copies(qw, copies)
    y = torch.empty((wl.M, wl.N), dtype=torch.float16, device="cuda")
    ws_bytes = wq.wq_gemm_workspace_bytes(wl.M, wl.N, wl.K, wl.group)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    t = _time_calls(lambda i: wq.wq_gemm_w4a16(xd, qws[i % copies], y=y, workspace=ws if ws_bytes else None),
                    steps, warmup)
    t_dense = _time_calls(lambda i: torch.matmul(xd, Wf.t()), max(10, steps // 4), 3)
    return wl, t, t_dense


def bench_quantize(wl_name="decode_gemv", reps=20):
    import torch
    import w4a16_bit_matmul_amd as wq
    import workloads
    wl = workloads.WORKLOADS[wl_name]
    Wd, _, qw = _quantize_workload(wl)
    t = _time_calls(lambda i: wq.wq_quantize_groups(Wd, wl.group, out=qw), reps, 3)
    qbytes, sbytes, zbytes = wq.wq_layout_bytes(wl.N, wl.K, wl.group)
    moved = wl.N * wl.K * 2 + qbytes + sbytes + zbytes
    return t, moved


def cpu_baseline(target_s=15.0):
    """The C oracle's fused product (dequantize + fp64 dot) on a bounded sample
    of the decode workload's rows, with all host threads."""
    import numpy as np
    import oracle
    import workloads
    wl = workloads.WORKLOADS["decode_gemv"]
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    rows = 256
    W = workloads.gen_weights(wl.w_seed, wl.N, wl.K, outlier_frac=wl.w_outlier_frac)[:4096]
    x = wl.activations()
    q, s, z = oracle.quantize_groups(W, wl.group, dtype=oracle.BF16)
    # grow the sample until the timed call takes a meaningful time
    while True:
        t0 = time.perf_counter()
        oracle.gemm_rows_f64(x, q, s, z, wl.group, 0, rows)
        dt = time.perf_counter() - t0
        if dt > target_s / 4 or rows >= q.shape[0]:
            break
        rows = min(q.shape[0], rows * 4)
    reps = max(1, int(target_s / max(dt, 1e-3)))
    reps = min(reps, 8)
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.gemm_rows_f64(x, q, s, z, wl.group, 0, rows)
    dt = (time.perf_counter() - t0) / reps
    frac = rows / wl.N
    bytes_sample = (wl.N * wl.K // 2 + 2 * wl.N * wl.K // wl.group + wl.N * wl.K // (2 * wl.group)) * frac \
        + 2 * wl.K + 2 * rows
    return {"value": round(bytes_sample / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"decode_gemv rows 0..{rows - 1} of {wl.N} (M=1, K={wl.K}, g={wl.group}), "
                      f"C oracle dequant + fp64 dot, {reps} reps, {dt:.2f}s each"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="time only the decode GEMV")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run an elementwise kernel over 256 MiB (reads and writes a known byte count), "
                         "to calibrate hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the W4A16 path here is a "
              f"single-GPU kernel library with no multi-GPU component", file=sys.stderr)
        sys.exit(2)
    _ensure_built()
    import torch
    torch.cuda.set_device(0)
    if args.copy_probe:
        a = torch.ones(64 << 20, dtype=torch.float32, device="cuda")  # 256 MiB
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b
        log("[bench] copy probe: 3 x elementwise neg over 256 MiB (268435456 B read, 268435456 B written)")

    wl, nbytes, copies, t_eager, t_graph, _ = bench_gemv(args.steps, args.warmup)
    log(f"[bench] decode GEMV: eager {t_eager * 1e6:.2f} us/call, graph {t_graph * 1e6:.2f} us/call, "
        f"{copies} weight copies")
    t_step = t_eager
    value = nbytes / t_step / 1e9
    achieved = nbytes / t_graph / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "M": wl.M, "N": wl.N, "K": wl.K, "group": wl.group,
                   "weights": "bf16 N(0,0.02), 0.1% input channels x20, quantized to INT4 on the GPU",
                   "activations": "fp16 N(0,1), 1% channels x10",
                   "algorithmic_bytes": nbytes, "weight_copies_rotated": copies,
                   "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "gemv_kernel<MT=1>", "timing": "hip events over graph-replayed back-to-back launches",
                     "us_per_launch": round(t_graph * 1e6, 3)},
    }
    if not args.no_extras:
        gwl, t_gemm, t_dense = bench_gemm(max(20, args.steps // 4), max(5, args.warmup // 4))
        tflops = gwl.flops() / t_gemm / 1e12
        line["gemm_m128"] = {"workload": gwl.name, "M": gwl.M, "N": gwl.N, "K": gwl.K, "group": gwl.group,
                             "us": round(t_gemm * 1e6, 2), "tflops": round(tflops, 2),
                             "frac_fp16_peak": round(tflops / FP16_PEAK_TFLOPS, 4),
                             "dense_fp16_torch_matmul_us": round(t_dense * 1e6, 2),
                             "dense_fp16_tflops": round(gwl.flops() / t_dense / 1e12, 2)}
        log(f"[bench] M=128 GEMM: {t_gemm * 1e6:.1f} us, {tflops:.1f} TFLOP/s; dense fp16 {t_dense * 1e6:.1f} us")
        tq, moved = bench_quantize()
        line["quantize"] = {"workload": "decode_gemv weights (bf16 8192x8192, g=128)", "us": round(tq * 1e6, 2),
                            "gbs": round(moved / tq / 1e9, 2)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
