"""Benchmark of the W4A16 hot path on one MI355X.

Step = one call of wq_gemm_w4a16 (the fused dequantize-and-multiply) on the
decode workload M=1, N=K=8192, group 128, with seeded synthetic bf16 weights
(quantized once on the GPU before timing) and fp16 activations, all resident
in HBM.  The weights are replicated into enough copies (>= 1 GB) that
consecutive steps never find them in the 256 MB last-level cache.

value = effective GB/s = algorithmic bytes (4-bit codes + fp16 scales + 4-bit
zero-points + fp16 x + fp16 y) / time per step.  The M=128 GEMM (TFLOP/s), the
quantization kernel and the CPU oracle are reported alongside in the same line.

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 200]
"""
from __future__ import annotations

import argparse
import ctypes
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
ROTATE_BYTES = 1024 << 20  # four times the 256 MB last-level cache
SETTLE_MS = 100.0          # untimed back-to-back launches before the headline's warm-up steps


def workloads_mod():
    import workloads
    return workloads


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


def _time_calls(fn, n_calls, warmup, sync_before=True):
    """Average time per call of n_calls back-to-back calls, from events on the
    launch stream (torch's current stream, the one libwq is handed)."""
    import torch
    for i in range(warmup):
        fn(i)
    if sync_before:
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n_calls):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / n_calls  # seconds per call


def read_clock(stream=None):
    """Core clock in MHz measured by the library's clock probe, launched now on
    the stream (after the work whose clock it reports) and synchronized: the
    median over 256 one-wave workgroups of the shader clock counter's advance
    per tick of the 100 MHz real-time counter, over a 20 us spin."""
    import torch
    import w4a16_bit_matmul_amd as wq
    out = wq.wq_clock_probe(256, 2000, stream=stream)
    torch.cuda.synchronize()
    c = out.cpu().double()
    mhz = (100.0 * c[:, 0] / c[:, 1]).median().item()
    return round(mhz, 1)


# One timing protocol for every figure beside the headline: warm-up launches
# of the same call until at least WARM_MS of GPU time (and at least
# WARM_MIN_LAUNCHES launches) have run, then a timed region of at least
# TIMED_MIN_LAUNCHES launches and TIMED_MIN_MS, between two HIP events on the
# launch stream, with the core clock read by the clock probe right before and
# right after the timed region.
WARM_MS = 40.0
WARM_MIN_LAUNCHES = 300
TIMED_MIN_LAUNCHES = 200
TIMED_MIN_MS = 20.0


def timed_protocol(run_batch, batch_launches, est_us=None):
    """run_batch() issues batch_launches back-to-back launches (one host call).
    Returns (seconds per launch, record of the protocol: warm-up and timed
    launch counts and the clock over the timed region)."""
    import torch
    if est_us is None:  # one batch to estimate the launch time
        est_us = _time_calls(lambda i: run_batch(), 1, 0) / batch_launches * 1e6
    warm_batches = max(1, math.ceil(max(WARM_MIN_LAUNCHES, WARM_MS * 1e3 / est_us) / batch_launches))
    timed_batches = max(1, math.ceil(max(TIMED_MIN_LAUNCHES, TIMED_MIN_MS * 1e3 / est_us) / batch_launches))
    for _ in range(warm_batches):
        run_batch()
    clk0 = read_clock()
    run_batch()  # keeps the GPU busy while the host issues the timed region
    t = _time_calls(lambda i: run_batch(), timed_batches, 0, sync_before=False) / batch_launches
    clk1 = read_clock()
    return t, {"warmup_launches": warm_batches * batch_launches, "timed_launches": timed_batches * batch_launches,
               "timing": "back-to-back launches between two HIP events on the launch stream",
               "clock_mhz_before": clk0, "clock_mhz_after": clk1}


def sha256_of(a) -> str:
    import hashlib
    return hashlib.sha256(a.tobytes()).hexdigest()


def _workspace(wl):
    import torch
    import w4a16_bit_matmul_amd as wq
    n = wq.wq_gemm_workspace_bytes(wl.M, wl.N, wl.K, wl.group)
    return torch.zeros(n, dtype=torch.uint8, device="cuda") if n else None


def bench_gemv(steps, warmup, name="decode_gemv"):
    import torch
    import w4a16_bit_matmul_amd as wq
    import workloads
    wl = workloads.WORKLOADS[name]
    Wd, xd, qw = _quantize_workload(wl)
    del Wd
    nbytes = wl.algorithmic_bytes()
    copies = max(2, math.ceil(ROTATE_BYTES / nbytes))
    qws = _device_copies(qw, copies)
    y = torch.empty((wl.M, wl.N), dtype=torch.float16, device="cuda")
    ws = _workspace(wl)

    # the timed steps are issued by one host call (wq_gemm_w4a16_seq, its
    # arguments marshalled before the timed region), so the GPU never waits
    # for the host; one Python call per step is timed alongside
    run_seq = wq.wq_gemm_w4a16_seq_prepared([xd] * steps, [qws[i % copies] for i in range(steps)], [y] * steps,
                                            workspace=ws)
    # Clock settling: the GPU's clocks settle only after tens of milliseconds
    # of sustained load, so before the warm-up steps the same product runs
    # back to back, untimed, for about SETTLE_MS (issued 1000 launches per
    # host call).  Then the `warmup` warm-up steps and, with no wait in
    # between, the `steps` timed steps, each group one wq_gemm_w4a16_seq call
    # (a timed region that began on an idle GPU would count the host's launch
    # latency).  The core clock is read by the clock probe right after the
    # timed region.
    n_settle = 1000
    settle = wq.wq_gemm_w4a16_seq_prepared([xd] * n_settle, [qws[i % copies] for i in range(n_settle)],
                                           [y] * n_settle, workspace=ws)
    t_settle_batch = _time_calls(lambda i: settle(), 1, 1)
    settle_batches = max(1, math.ceil(SETTLE_MS * 1e-3 / t_settle_batch))
    # no synchronization from here to the end of the timed steps: the settling
    # launches still queued keep the GPU busy while the host records the first
    # event and issues the timed steps, so the timed region never waits for the
    # host
    for _ in range(settle_batches):
        settle()
    warm = None
    if warmup > 0:
        warm = wq.wq_gemm_w4a16_seq_prepared([xd] * warmup, [qws[(steps + i) % copies] for i in range(warmup)],
                                             [y] * warmup, workspace=ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if warm is not None:
        warm()
    e0.record()
    run_seq()
    e1.record()
    clock_mhz = read_clock()
    t_step = e0.elapsed_time(e1) / 1e3 / steps
    t_single = _time_calls(lambda i: wq.wq_gemm_w4a16(xd, qws[i % copies], y=y, workspace=ws), steps, 0)
    clock = {"clock_mhz_after_timed_steps": clock_mhz,
             "settle_launches_before_warmup": (settle_batches + 1) * n_settle,
             "source": "clock probe (s_memtime against the 100 MHz s_memrealtime), launched right after the timed steps"}
    return wl, nbytes, copies, t_step, t_single, clock


def flush_check(calls=200, warmup=2000):
    """Cross-check of the weight rotation: the decode GEMV on ONE weight copy,
    with a 512 MiB read-and-write flush of the GPU's caches (256 MB last-level
    cache) between consecutive calls, each call timed alone by events on the
    launch stream; next to the same calls back to back without the flush (the
    weights then stay cache resident) and the rotated figure of bench_gemv."""
    import statistics
    import torch
    import w4a16_bit_matmul_amd as wq
    import workloads
    wl = workloads.WORKLOADS["decode_gemv"]
    Wd, xd, qw = _quantize_workload(wl)
    del Wd
    y = torch.empty((wl.M, wl.N), dtype=torch.float16, device="cuda")
    ws = _workspace(wl)
    scratch = torch.zeros(128 << 20, dtype=torch.float32, device="cuda")  # 512 MiB
    for _ in range(warmup):
        wq.wq_gemm_w4a16(xd, qw, y=y, workspace=ws)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for e0, e1 in ev:
        scratch.add_(1.0)  # reads and writes 512 MiB: evicts the weights from every cache level
        e0.record()
        wq.wq_gemm_w4a16(xd, qw, y=y, workspace=ws)
        e1.record()
    torch.cuda.synchronize()
    flushed = [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]
    hot = _time_calls(lambda i: wq.wq_gemm_w4a16(xd, qw, y=y, workspace=ws), calls, 0) * 1e6
    return {"workload": "decode_gemv", "calls": calls, "flush_bytes": 512 << 20,
            "us_per_call_flushed_median": round(statistics.median(flushed), 3),
            "us_per_call_flushed_mean": round(statistics.mean(flushed), 3),
            "us_per_call_same_copy_back_to_back": round(hot, 3),
            "note": "flushed calls are timed one at a time (each includes one event pair's overhead); the "
                    "rotated back-to-back figure is the benchmark value"}


def bench_dense_same_shape():
    """Dense fp16 torch.matmul of the batched workload's shape (fp16 weights
    of 470 MB, larger than the last-level cache), under the common protocol."""
    import numpy as np
    import torch
    import workloads
    wl = workloads.WORKLOADS["batched_gemm"]
    Wf = torch.from_numpy(wl.weights().view(np.int16)).cuda().view(torch.bfloat16).to(torch.float16)
    xd = torch.from_numpy(wl.activations().view(np.int16)).cuda().view(torch.float16)
    Wt = Wf.t()
    t, proto = timed_protocol(lambda: torch.matmul(xd, Wt), 1)
    del Wf, Wt
    return t, proto


def bench_w8(steps, warmup):
    """Group absmax int8 weights (W8A16) on the decode and M=128 workloads:
    the same seeded weights quantized to int8 on the GPU, the GEMV and the MFMA
    GEMM timed like the 4-bit ones (one Python call per launch; the int8 GEMV
    takes longer than that call)."""
    import numpy as np
    import torch
    import w4a16_bit_matmul_amd as wq
    import workloads
    out = {}
    for name in ("decode_gemv", "batched_gemm"):
        wl = workloads.WORKLOADS[name]
        W = wl.weights()
        Wd = torch.from_numpy(W.view(np.int16)).cuda().view(torch.bfloat16)
        xd = torch.from_numpy(wl.activations().view(np.int16)).cuda().view(torch.float16)
        qw = wq.wq_quantize_w8(Wd, wl.group)["qw"]
        del Wd
        nbytes = wl.algorithmic_bytes_w8()
        copies = max(2, math.ceil(ROTATE_BYTES / nbytes))
        qws = [qw] + [wq.QuantizedWeight8(qw.qpacked.clone(), qw.s.clone(), qw.N, qw.K, qw.group)
                      for _ in range(copies - 1)]
        y = torch.empty((wl.M, wl.N), dtype=torch.float16, device="cuda")
        n = wq.wq_gemm_w8a16_workspace_bytes(wl.M, wl.N, wl.K, wl.group)
        ws = torch.zeros(n, dtype=torch.uint8, device="cuda") if n else None
        nb = max(copies, 20)
        t, proto = timed_protocol(lambda: [wq.wq_gemm_w8a16(xd, qws[i % copies], y=y, workspace=ws)
                                           for i in range(nb)], nb)
        rec = {"workload": wl.name, "M": wl.M, "N": wl.N, "K": wl.K, "group": wl.group,
               "kernel": wq.wq_gemm_w8a16_plan(wl.M, wl.N, wl.K, wl.group), "us_per_launch": round(t * 1e6, 3),
               "algorithmic_bytes": nbytes, "gbs": round(nbytes / t / 1e9, 2),
               "frac_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4), "weight_copies_rotated": copies,
               "launches": "one Python call each", **proto}
        if wl.M >= 64:
            tf = wl.flops() / t / 1e12
            rec.update({"tflops": round(tf, 2), "frac_fp16_peak": round(tf / FP16_PEAK_TFLOPS, 4)})
        out[name] = rec
        log(f"[bench] W8A16 {name}: {t * 1e6:.2f} us per launch, {nbytes / t / 1e9:.1f} GB/s")
    return out


def bench_kv(steps, warmup):
    """INT4 KV cache in blocks of 128, the 70B layer's K and V (8 KV heads x
    128 = 1024 values per token): the decode append (64 sequences, K and V
    rows of one layer stacked: 128 rows scattered into a 131072-row cache) and
    a 32768-token prefill of one K tensor (bf16 in)."""
    import numpy as np
    import torch
    import w4a16_bit_matmul_amd as wq
    import workloads
    hd = 1024
    out = {}
    rng = np.random.default_rng(77)
    for name, T, S in (("decode_append", 128, 131072), ("prefill", 32768, 32768)):
        X = workloads.f32_to_bf16_bits(rng.standard_normal((T, hd)).astype(np.float32))
        Xd = torch.from_numpy(X.view(np.int16)).cuda().view(torch.bfloat16)
        cache = wq.kv_cache_alloc(S, hd)
        slot = None
        if name == "decode_append":
            slot = torch.from_numpy(rng.choice(S, T, replace=False).astype(np.int32)).cuda()
        # arguments marshalled once: each timed call is one C call (the append
        # is shorter than a Python call of the binding)
        fn = wq.lib().wq_kv_quantize
        args = (ctypes.c_void_p(Xd.data_ptr()), wq.WQ_BF16, T, hd,
                None if slot is None else ctypes.c_void_p(slot.data_ptr()), S, ctypes.c_void_p(cache.codes.data_ptr()),
                ctypes.c_void_p(cache.s.data_ptr()), ctypes.c_void_p(cache.zpacked.data_ptr()),
                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert fn(*args) == wq.WQ_OK
        nb = 50
        t, proto = timed_protocol(lambda: [fn(*args) for _ in range(nb)], nb)
        moved = T * hd * 2 + T * hd // 2 + T * (hd // 128) * 2 + T * ((hd // 128 + 1) // 2) + (T * 4 if slot is not None else 0)
        out[name] = {"tokens": T, "values_per_token": hd, "cache_rows": S, "us_per_call": round(t * 1e6, 3),
                     "bytes": moved, "gbs": round(moved / t / 1e9, 2),
                     "frac_hbm_peak": round(moved / t / 1e9 / HBM_PEAK_GBS, 4), **proto}
        log(f"[bench] KV int4 {name}: {t * 1e6:.2f} us per call, {moved / t / 1e9:.1f} GB/s")
    return out


def bench_mxfp4(steps, warmup):
    """MXFP4 weights (E2M1, blocks of 32, E8M0 scales) on the decode and M=128
    workloads, timed like the int8 leg; plus each format's weight error on the
    decode layer (relative Frobenius norm of W_hat - W)."""
    import numpy as np
    import torch
    import w4a16_bit_matmul_amd as wq
    import workloads
    out = {}
    for name in ("decode_gemv", "batched_gemm"):
        wl = workloads.WORKLOADS[name]
        Wd = torch.from_numpy(wl.weights().view(np.int16)).cuda().view(torch.bfloat16)
        xd = torch.from_numpy(wl.activations().view(np.int16)).cuda().view(torch.float16)
        qw = wq.wq_quantize_mxfp4(Wd)["qw"]
        if name == "decode_gemv":
            ref = Wd.float()
            nrm = float(ref.norm())
            err = {"mxfp4_g32": float((wq.wq_dequant_mxfp4(qw) - ref).norm()) / nrm}
            for g in (32, 128):
                err[f"int4_asym_g{g}"] = float((wq.wq_dequant(wq.wq_quantize_groups(Wd, g)["qw"]) - ref).norm()) / nrm
            out["weight_relative_error"] = {k: round(v, 5) for k, v in err.items()}
        del Wd
        nbytes = wl.N * wl.K // 2 + wl.N * wl.K // 32 + 2 * wl.M * wl.K + 2 * wl.M * wl.N
        copies = max(2, math.ceil(ROTATE_BYTES / nbytes))
        qws = [qw] + [wq.QuantizedWeightMX(qw.qpacked.clone(), qw.e8.clone(), qw.N, qw.K) for _ in range(copies - 1)]
        y = torch.empty((wl.M, wl.N), dtype=torch.float16, device="cuda")
        n = wq.wq_gemm_mxfp4_workspace_bytes(wl.M, wl.N, wl.K)
        ws = torch.zeros(n, dtype=torch.uint8, device="cuda") if n else None
        nb = max(copies, 20)
        t, proto = timed_protocol(lambda: [wq.wq_gemm_mxfp4(xd, qws[i % copies], y=y, workspace=ws)
                                           for i in range(nb)], nb)
        rec = {"workload": wl.name, "M": wl.M, "N": wl.N, "K": wl.K, "kernel": wq.wq_gemm_mxfp4_plan(wl.M, wl.N, wl.K),
               "us_per_launch_one_python_call_each": round(t * 1e6, 3), "algorithmic_bytes": nbytes,
               "gbs": round(nbytes / t / 1e9, 2), "frac_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
               "weight_copies_rotated": copies, **proto}
        if wl.M >= 64:
            tf = wl.flops() / t / 1e12
            rec.update({"tflops": round(tf, 2), "frac_fp16_peak": round(tf / FP16_PEAK_TFLOPS, 4)})
        out[name] = rec
        log(f"[bench] MXFP4 {name}: {t * 1e6:.2f} us per launch, {nbytes / t / 1e9:.1f} GB/s")
    return out


def bench_nvfp4(steps, warmup):
    """NVFP4 weights (E2M1, blocks of 16, E4M3 scales, fp32 tensor scale) on the
    decode and M=128 workloads, timed like the MXFP4 leg, with the weight error
    on the decode layer (relative Frobenius norm of W_hat - W)."""
    import numpy as np
    import torch
    import w4a16_bit_matmul_amd as wq
    import workloads
    out = {}
    for name in ("decode_gemv", "batched_gemm"):
        wl = workloads.WORKLOADS[name]
        Wd = torch.from_numpy(wl.weights().view(np.int16)).cuda().view(torch.bfloat16)
        xd = torch.from_numpy(wl.activations().view(np.int16)).cuda().view(torch.float16)
        qw = wq.wq_quantize_nvfp4(Wd)["qw"]
        if name == "decode_gemv":
            ref = Wd.float()
            out["weight_relative_error_nvfp4_g16"] = round(float((wq.wq_dequant_nvfp4(qw) - ref).norm()) /
                                                           float(ref.norm()), 5)
        del Wd
        nbytes = wl.N * wl.K // 2 + wl.N * wl.K // 16 + 4 + 2 * wl.M * wl.K + 2 * wl.M * wl.N
        copies = max(2, math.ceil(ROTATE_BYTES / nbytes))
        qws = [qw] + [wq.QuantizedWeightNV(qw.qpacked.clone(), qw.s8.clone(), qw.tensor_scale.clone(), qw.N, qw.K)
                      for _ in range(copies - 1)]
        y = torch.empty((wl.M, wl.N), dtype=torch.float16, device="cuda")
        n = wq.wq_gemm_nvfp4_workspace_bytes(wl.M, wl.N, wl.K)
        ws = torch.zeros(n, dtype=torch.uint8, device="cuda") if n else None
        nb = max(copies, 20)
        t, proto = timed_protocol(lambda: [wq.wq_gemm_nvfp4(xd, qws[i % copies], y=y, workspace=ws)
                                           for i in range(nb)], nb)
        rec = {"workload": wl.name, "M": wl.M, "N": wl.N, "K": wl.K, "kernel": wq.wq_gemm_nvfp4_plan(wl.M, wl.N, wl.K),
               "us_per_launch_one_python_call_each": round(t * 1e6, 3), "algorithmic_bytes": nbytes,
               "gbs": round(nbytes / t / 1e9, 2), "frac_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
               "weight_copies_rotated": copies, **proto}
        if wl.M >= 64:
            tf = wl.flops() / t / 1e12
            rec.update({"tflops": round(tf, 2), "frac_fp16_peak": round(tf / FP16_PEAK_TFLOPS, 4)})
        out[name] = rec
        log(f"[bench] NVFP4 {name}: {t * 1e6:.2f} us per launch, {nbytes / t / 1e9:.1f} GB/s")
    return out


def bench_awq():
    """AWQ-style fold on the decode layer (8192 x 8192, g=128): salient channels
    = the 1 % with the largest mean |x| over 64 calibration rows (the library's
    statistic), alpha = factor there; the error ||y - x W^T|| of the INT4
    product over 64 evaluation rows (same outlier channels, other values),
    against the fp32 product of the unquantized bf16 weights, for each factor;
    and the time of the activation-side kernel at M = 1."""
    import numpy as np
    import torch
    import w4a16_bit_matmul_amd as wq
    import workloads
    wl = workloads.WORKLOADS["decode_gemv"]
    Wd = torch.from_numpy(wl.weights().view(np.int16)).cuda().view(torch.bfloat16)
    f16 = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.float16)
    x = f16(workloads.gen_activations(wl.x_seed, 64, wl.K, outlier_frac=wl.x_outlier_frac))
    x_cal = f16(workloads.gen_activations(wl.x_seed + 50, 64, wl.K, outlier_frac=wl.x_outlier_frac,
                                          channel_seed=wl.x_seed + 1))
    y_true = (x.float() @ Wd.float().t()).double()
    stat = wq.wq_channel_absmean(x_cal)
    top = torch.argsort(stat, descending=True, stable=True)[:round(0.01 * wl.K)]
    err = {}
    for factor in (1.0, 1.5, 2.0, 3.0, 4.0):
        alpha = torch.ones(wl.K, dtype=torch.float32, device="cuda")
        alpha[top] = factor
        qw = wq.wq_quantize_groups(Wd, wl.group, alpha=alpha)["qw"]
        y = wq.wq_gemm_w4a16(wq.wq_scale_activations(x, alpha), qw)
        err[factor] = float((y.double() - y_true).norm())
    alpha = torch.ones(wl.K, dtype=torch.float32, device="cuda")
    x1 = x[:1].contiguous()
    out = torch.empty_like(x1)
    t = _time_calls(lambda i: wq.wq_scale_activations(x1, alpha, out=out), 200, 200)
    best = min((f for f in err if f != 1.0), key=lambda f: err[f])
    log(f"[bench] AWQ fold: error ratio {err[best] / err[1.0]:.3f} at factor {best}; activation scaling {t * 1e6:.2f} us")
    return {"workload": "decode_gemv layer, 64 calibration + 64 evaluation rows", "salient_channels": int(top.numel()),
            "error_norm_by_factor": {str(k): round(v, 5) for k, v in err.items()},
            "best_factor": best, "error_ratio_best": round(err[best] / err[1.0], 4),
            "scale_activations_us_m1_python_call": round(t * 1e6, 3)}


def bench_sweep(steps):
    """Every workload (the tiny case, decode, the M=16 up-projection, the M=128
    GEMM and the g=32 sweep of 70B layer shapes) through both kernel families:
    time per launch, effective GB/s and TFLOP/s; one JSON line each."""
    import numpy as np
    import torch
    import w4a16_bit_matmul_amd as wq
    import workloads
    qcache = {}
    for name, wl in workloads.WORKLOADS.items():
        key = (wl.w_seed, wl.N, wl.K, wl.group, wl.w_dtype)
        if key not in qcache:
            qcache.clear()
            W = wl.weights()
            Wd = torch.from_numpy(W.view(np.int16 if W.dtype == np.uint16 else np.float32)).cuda()
            if W.dtype == np.uint16:
                Wd = Wd.view(torch.bfloat16)
            qw = wq.wq_quantize_groups(Wd, wl.group)["qw"]
            del Wd
            copies = max(2, math.ceil(ROTATE_BYTES / wl.algorithmic_bytes()))
            qcache[key] = _device_copies(qw, copies)
        qws = qcache[key]
        copies = len(qws)
        xd = torch.from_numpy(wl.activations().view(np.int16)).cuda().view(torch.float16)
        y = torch.empty((wl.M, wl.N), dtype=torch.float16, device="cuda")
        ws = _workspace(wl)
        rec = {"workload": name, "M": wl.M, "N": wl.N, "K": wl.K, "group": wl.group,
               "auto": "mfma" if wq.auto_uses_mfma(wl.M, wl.N, "int4", wl.K, wl.group) else "gemv"}
        for path, tag in ((wq.WQ_PATH_GEMV, "gemv"), (wq.WQ_PATH_MFMA, "mfma")):
            n_steps = max(20, steps // 4)
            t = _time_calls(lambda i: wq.wq_gemm_w4a16(xd, qws[i % copies], y=y, workspace=ws, path=path), n_steps,
                            max(50, 2000 // max(1, wl.M)))
            rec[tag] = {"us": round(t * 1e6, 3), "gbs": round(wl.algorithmic_bytes() / t / 1e9, 1),
                        "tflops": round(wl.flops() / t / 1e12, 2)}
        print(json.dumps(rec), flush=True)


def bench_read_ceiling(nbytes, steps, warmup):
    """The streaming-read probe on the decode GEMV's byte count (rounded up to
    256), rotating over >= 1 GB so that every launch reads HBM: the best of
    1, 2, 4 and 8 16-byte loads per thread, plain or non-temporal.  Each timed
    run is one C call that issues every launch, so the host never gaps the GPU.
    Then one launch reading 1 GiB at once (four times the last-level cache),
    under the common protocol: its rate is the steady-state read bandwidth,
    and the decode-sized read's time minus its bytes at that rate is the
    per-launch fixed cost (launch, ramp, drain)."""
    import torch
    import w4a16_bit_matmul_amd as wq
    window = (nbytes + 255) // 256 * 256
    nwin = max(2, math.ceil(ROTATE_BYTES / window))
    buf = torch.ones(window * nwin // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    best = None
    for nt in (False, True):
        for chunks in (1, 2, 4, 8):
            wq.wq_read_probe(buf, window, warmup, chunks=chunks, nontemporal=nt, sink=sink)
            t = _time_calls(lambda i: wq.wq_read_probe(buf, window, steps, chunks=chunks, nontemporal=nt, sink=sink),
                            1, 0) / steps
            if best is None or t < best[0]:
                best = (t, chunks, nt)
    del buf
    t, chunks, nt = best
    rec = {"bytes_per_launch": window, "us_per_launch": round(t * 1e6, 3), "gbs": round(window / t / 1e9, 2),
           "frac_hbm_peak": round(window / t / 1e9 / HBM_PEAK_GBS, 4), "loads_per_thread": chunks,
           "nontemporal": nt, "windows_rotated": nwin}
    big = 1 << 30
    buf = torch.ones(big // 4, dtype=torch.int32, device="cuda")
    best_big = None
    for chunks in (2, 4, 8):
        tb, proto = timed_protocol(lambda: wq.wq_read_probe(buf, big, 1, chunks=chunks, nontemporal=True, sink=sink), 1)
        if best_big is None or tb < best_big[0]:
            best_big = (tb, chunks, proto)
    del buf
    tb, chunks_b, proto = best_big
    bw = big / tb
    rec["one_launch_1gib"] = {"bytes": big, "us_per_launch": round(tb * 1e6, 2), "gbs": round(bw / 1e9, 1),
                              "frac_hbm_peak": round(bw / 1e9 / HBM_PEAK_GBS, 4), "loads_per_thread": chunks_b,
                              "nontemporal": True, **proto}
    rec["fixed_cost_us_at_decode_size"] = round((t - window / bw) * 1e6, 3)
    log(f"[bench] read ceiling: {window} B in {t * 1e6:.2f} us; 1 GiB in one launch {tb * 1e6:.1f} us "
        f"({bw / 1e9:.0f} GB/s); fixed cost {rec['fixed_cost_us_at_decode_size']} us")
    return rec


def bench_configs():
    """Every workload (the tiny case, decode, the M=16 up-projection, the M=128
    GEMM and the g=32 sweep of 70B layer shapes) on the kernel WQ_PATH_AUTO
    picks, under the common timing protocol (timed_protocol): launches issued
    by wq_gemm_w4a16_seq calls (arguments marshalled beforehand, so the host
    never gaps the GPU), weights rotated over >= 1 GB of copies (at most 128);
    effective GB/s and TFLOP/s, the inputs' SHA-256 and the clock.  The M=16
    up-projection, which WQ_PATH_AUTO runs on the split-K GEMV, is also timed
    on the MFMA GEMM kernel (forced)."""
    import numpy as np
    import torch
    import w4a16_bit_matmul_amd as wq
    import workloads
    out = {}
    qcache = {}
    for name, wl in workloads.WORKLOADS.items():
        key = (wl.w_seed, wl.N, wl.K, wl.group, wl.w_dtype)
        if key not in qcache:
            qcache.clear()
            torch.cuda.empty_cache()
            W = wl.weights()
            w_sha = sha256_of(W)
            if W.dtype == np.uint16:
                Wd = torch.from_numpy(W.view(np.int16)).cuda().view(torch.bfloat16)
            else:
                Wd = torch.from_numpy(W).cuda()
            qw = wq.wq_quantize_groups(Wd, wl.group)["qw"]
            del Wd, W
            copies = min(128, max(2, math.ceil(ROTATE_BYTES / wl.algorithmic_bytes())))
            qcache[key] = (_device_copies(qw, copies), w_sha)
        qws, w_sha = qcache[key]
        copies = len(qws)
        x = wl.activations()
        xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.float16)
        y = torch.empty((wl.M, wl.N), dtype=torch.float16, device="cuda")
        ws = _workspace(wl)
        nbytes = wl.algorithmic_bytes()
        n = max(copies, 50)
        paths = [("auto", wq.WQ_PATH_AUTO)]
        if name == "mlp_up_decode":
            paths.append(("forced_mfma", wq.WQ_PATH_MFMA))
        for tag, path in paths:
            if path == wq.WQ_PATH_AUTO:
                run_seq = wq.wq_gemm_w4a16_seq_prepared([xd] * n, [qws[i % copies] for i in range(n)], [y] * n,
                                                        workspace=ws)
            else:  # one Python call per launch: a forced path has no sequence entry point
                wsg = torch.zeros(max(1, wq.wq_gemm_workspace_bytes(wl.M, wl.N, wl.K, wl.group, path)),
                                  dtype=torch.uint8, device="cuda")
                run_seq = lambda: [wq.wq_gemm_w4a16(xd, qws[i % copies], y=y, workspace=wsg, path=path)
                                   for i in range(n)]
            t, proto = timed_protocol(run_seq, n)
            rec = {"M": wl.M, "N": wl.N, "K": wl.K, "group": wl.group,
                   "kernel": wq.wq_gemm_plan(wl.M, wl.N, wl.K, wl.group, path), "us_per_launch": round(t * 1e6, 3),
                   "algorithmic_bytes": nbytes, "gbs": round(nbytes / t / 1e9, 1),
                   "frac_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
                   "tflops": round(wl.flops() / t / 1e12, 2),
                   "frac_fp16_peak": round(wl.flops() / t / 1e12 / FP16_PEAK_TFLOPS, 4),
                   "weight_copies_rotated": copies, **proto, "W_sha256": w_sha, "x_sha256": sha256_of(x)}
            if tag == "auto":
                out[name] = rec
            else:
                out[name][tag] = rec
            log(f"[bench] {name} ({tag}): {t * 1e6:.2f} us per launch, {nbytes / t / 1e9:.0f} GB/s, "
                f"{wl.flops() / t / 1e12:.1f} TFLOP/s, clock {proto.get('clock_mhz_after')} MHz")
    return out


def bench_matrix_ceiling():
    """The matrix-core counterpart of the read ceiling: the library's MFMA
    probe (v_mfma_f32_16x16x32_f16 on register operands, nothing else) on 1024
    workgroups of four waves, and a compute-bound dense fp16 GEMM
    (torch.matmul, hipBLASLt, 8192 x 8192 x 8192), each under the common
    protocol with the clock sampled."""
    import torch
    import w4a16_bit_matmul_amd as wq
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    wgs, iters, per_batch = 1024, 1024, 10
    flop = wq.wq_mfma_probe(wgs, iters, 1, sink=sink)
    t, proto = timed_protocol(lambda: wq.wq_mfma_probe(wgs, iters, per_batch, sink=sink), per_batch)
    probe = {"instruction": "v_mfma_f32_16x16x32_f16", "flop_per_launch": flop, "us_per_launch": round(t * 1e6, 2),
             "tflops": round(flop / t / 1e12, 1), "frac_fp16_peak": round(flop / t / 1e12 / FP16_PEAK_TFLOPS, 4),
             "grid": f"{wgs} workgroups x 256 threads, {iters} x 8 MFMAs per wave", **proto}
    n = 8192
    a = torch.randn((n, n), dtype=torch.float16, device="cuda")
    b = torch.randn((n, n), dtype=torch.float16, device="cuda")
    c = torch.empty((n, n), dtype=torch.float16, device="cuda")
    t2, proto2 = timed_protocol(lambda: torch.matmul(a, b, out=c), 1)
    dense = {"shape": [n, n, n], "us_per_call": round(t2 * 1e6, 1), "tflops": round(2 * n ** 3 / t2 / 1e12, 1),
             "frac_fp16_peak": round(2 * n ** 3 / t2 / 1e12 / FP16_PEAK_TFLOPS, 4), **proto2}
    del a, b, c
    log(f"[bench] matrix ceiling: MFMA probe {probe['tflops']} TFLOP/s at {probe.get('clock_mhz_after')} MHz; "
        f"dense fp16 GEMM 8192^3 {dense['tflops']} TFLOP/s")
    return {"mfma_probe": probe, "dense_fp16_gemm_8192": dense}


def bench_quantize(wl_name="decode_gemv", reps=20):
    import torch
    import w4a16_bit_matmul_amd as wq
    import workloads
    wl = workloads.WORKLOADS[wl_name]
    Wd, _, qw = _quantize_workload(wl)
    t, _ = timed_protocol(lambda: wq.wq_quantize_groups(Wd, wl.group, out=qw), 1)
    qbytes, sbytes, zbytes = wq.wq_layout_bytes(wl.N, wl.K, wl.group)
    moved = wl.N * wl.K * 2 + qbytes + sbytes + zbytes
    return t, moved


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemv_decode_m1_n8192_k8192_g128_hbm_traffic.md")
KERNEL_SOURCES = ("w4a16_bit_matmul_amd/csrc/wq_gemv.hip", "w4a16_bit_matmul_amd/csrc/wq_device.h")


def kernel_source_digest():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the decode GEMV from the committed rocprofv3
    counter summary (L2-to-memory read requests weighted by their size, and
    WRITE_SIZE, each scaled by the factor a copy kernel of known size gives),
    or None when that summary is missing or was taken on other kernel sources
    than the ones built now."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            fields = dict(ln[2:].split(": ", 1) for ln in f.read().splitlines() if ln.startswith("- ") and ": " in ln)
        if fields.get("kernel_source_sha256", "").strip("` ") != kernel_source_digest():
            return None
        return int(fields["traffic_bytes_per_launch"].strip("` "))
    except (OSError, KeyError, ValueError):
        return None


def _oracle_rate(fn, nbytes, target_s):
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= target_s:
            break
    return nbytes * reps / dt / 1e9, reps, dt


def cpu_baseline(target_s=12.0, leg_s=3.0):
    """The C oracle timed on the host: its fused product (dequantize each
    weight row, fp64 dot with x) over the whole decode workload for about
    target_s seconds on all host threads, reported in the metric's unit
    (algorithmic GB/s); beside it, legs of about leg_s seconds each: the
    product on one thread, and the oracle's quantization of the same weights
    (bf16 read, codes, scales and zero-points written) on all threads and on
    one."""
    import oracle
    import workloads
    wl = workloads.WORKLOADS["decode_gemv"]
    threads = len(os.sched_getaffinity(0))
    W = wl.weights()
    x = wl.activations()
    oracle.set_threads(threads)
    q, s, z = oracle.quantize_groups(W, wl.group, dtype=oracle.BF16)
    nbytes = wl.algorithmic_bytes()
    product = lambda: oracle.gemm_rows_f64(x, q, s, z, wl.group, 0, wl.N)
    rate, reps, dt = _oracle_rate(product, nbytes, target_s)
    qbytes = wl.N * wl.K * 2 + wl.N * wl.K // 2 + wl.N * (wl.K // wl.group) * 2 + wl.N * (wl.K // wl.group + 1) // 2
    quant = lambda: oracle.quantize_groups(W, wl.group, dtype=oracle.BF16)
    legs = {}
    for tag, n in (("all_threads", threads), ("one_thread", 1)):
        oracle.set_threads(n)
        if n == 1:
            r, k, d = _oracle_rate(product, nbytes, leg_s)
            legs[f"product_{tag}"] = {"gbs": round(r, 4), "threads": n, "reps": k, "seconds": round(d, 2)}
        r, k, d = _oracle_rate(quant, qbytes, leg_s)
        legs[f"quantize_{tag}"] = {"gbs": round(r, 4), "threads": n, "reps": k, "seconds": round(d, 2),
                                   "bytes": qbytes}
    oracle.set_threads(threads)
    legs["product_all_threads"] = {"gbs": round(rate, 4), "threads": threads, "reps": reps, "seconds": round(dt, 2)}
    return {"value": round(rate, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"whole decode_gemv product (M=1, N=K={wl.K}, g={wl.group}): C oracle dequantizes each "
                      f"row and takes fp64 dot products, {reps} repetitions in {dt:.1f}s "
                      f"({dt / reps * 1e3:.1f} ms each), {threads} OpenMP threads; legs: the same product on one "
                      f"thread, and the oracle's quantization of the same 8192x8192 bf16 weights on all threads "
                      f"and on one (GB/s of bf16 in + codes, scales, zero-points out), about {leg_s:.0f} s each",
            "legs": legs}


def main():
    global ROTATE_BYTES
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # warm-up steps after the ~100 ms of untimed clock settling
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="time only the decode GEMV")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the benchmark line, time every workload through both kernel families "
                         "(one JSON line each)")
    ap.add_argument("--flush-check", action="store_true",
                    help="instead of the benchmark line, time the decode GEMV on one weight copy with a 512 MiB "
                         "cache flush between calls (cross-check of the weight rotation)")
    ap.add_argument("--rotate-mb", type=int, default=ROTATE_BYTES >> 20,
                    help="span of the weight copies the timed calls rotate over, in MiB (default 1024, four "
                         "times the last-level cache)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run an elementwise kernel over 256 MiB (reads and writes a known byte count), "
                         "to calibrate hardware byte counters")
    args = ap.parse_args()
    ROTATE_BYTES = args.rotate_mb << 20
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

    import w4a16_bit_matmul_amd as wq
    if args.sweep:
        bench_sweep(args.steps)
        return
    if args.flush_check:
        rec = flush_check()
        _, _, copies, t_step, _, _ = bench_gemv(args.steps, args.warmup)
        rec["us_per_call_rotated_back_to_back"] = round(t_step * 1e6, 3)
        rec["rotated_weight_copies"] = copies
        rec["rotate_mb"] = args.rotate_mb
        print(json.dumps(rec), flush=True)
        return
    wl, nbytes, copies, t_step, t_single, clock = bench_gemv(args.steps, args.warmup)
    plan = wq.wq_gemm_plan(wl.M, wl.N, wl.K, wl.group)
    log(f"[bench] decode GEMV: {t_step * 1e6:.2f} us per launch back to back "
        f"(one Python call per launch: {t_single * 1e6:.2f} us), {copies} weight copies; {plan}")
    # one step is one launch of the GEMV kernel: the step rate and the kernel's
    # average launch duration are the same measurement
    value = nbytes / t_step / 1e9
    achieved = value
    traffic = measured_traffic()
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
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 TCC_EA0_RDREQ_{32B,64B,128B} x size + WRITE_SIZE, "
                                     "copy-calibrated)",
                     "traffic_over_algorithmic": None if traffic is None else round(traffic / nbytes, 4),
                     "algorithmic_bytes_per_launch": nbytes,
                     "kernel": plan,
                     "timing": f"{args.steps} back-to-back launches (one wq_gemm_w4a16_seq call) between two "
                               f"HIP events on the launch stream",
                     "us_per_launch": round(t_step * 1e6, 3),
                     "us_per_launch_one_python_call_each": round(t_single * 1e6, 3),
                     "clock": clock},
    }
    line["config"].update(W_sha256=sha256_of(wl.weights()), x_sha256=sha256_of(wl.activations()))
    if not args.no_extras:
        # every other figure below follows one timing protocol (timed_protocol):
        # >= 40 ms and >= 300 launches of warm-up, then >= 200 launches and
        # >= 20 ms timed, the clock sampled over the timed region
        line["configs"] = bench_configs()
        bg = line["configs"]["batched_gemm"]
        t_dense, proto_dense = bench_dense_same_shape()
        ceiling = bench_matrix_ceiling()
        gwl = workloads_mod().WORKLOADS["batched_gemm"]
        line["gemm_m128"] = {"workload": gwl.name, "M": gwl.M, "N": gwl.N, "K": gwl.K, "group": gwl.group,
                             "kernel": bg["kernel"], "bound": "mfma", "us_per_launch": bg["us_per_launch"],
                             "tflops": bg["tflops"], "peak_tflops": FP16_PEAK_TFLOPS,
                             "frac_fp16_peak": bg["frac_fp16_peak"],
                             "frac_of_mfma_probe": round(bg["tflops"] / ceiling["mfma_probe"]["tflops"], 4),
                             "source": "the batched_gemm entry of configs (same measurement)",
                             "warmup_launches": bg["warmup_launches"], "timed_launches": bg["timed_launches"],
                             "clock_mhz_after": bg.get("clock_mhz_after"),
                             "dense_fp16_torch_matmul_us": round(t_dense * 1e6, 2),
                             "dense_fp16_tflops": round(gwl.flops() / t_dense / 1e12, 2),
                             "dense_fp16_protocol": proto_dense}
        line["matrix_ceiling"] = ceiling
        log(f"[bench] M=128 GEMM: {bg['us_per_launch']:.1f} us per launch, {bg['tflops']:.1f} TFLOP/s; "
            f"dense fp16 {t_dense * 1e6:.1f} us")
        tq, moved = bench_quantize()
        line["quantize"] = {"workload": "decode_gemv weights (bf16 8192x8192, g=128)", "us": round(tq * 1e6, 2),
                            "gbs": round(moved / tq / 1e9, 2)}
        line["w8a16"] = bench_w8(args.steps, args.warmup)
        line["kv_int4"] = bench_kv(args.steps, args.warmup)
        line["awq_fold"] = bench_awq()
        line["mxfp4"] = bench_mxfp4(args.steps, args.warmup)
        line["nvfp4"] = bench_nvfp4(args.steps, args.warmup)
        line["read_ceiling"] = bench_read_ceiling(nbytes, max(200, args.steps), 2000)
        line["read_ceiling"]["gemv_frac_of_ceiling"] = round(line["read_ceiling"]["us_per_launch"] / (t_step * 1e6), 4)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
