"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (the default kernel choice): codes, scales, zero-points and
both packed layouts bit-exact against the oracle over the whole matrix; the
product on every output, against the oracle's product over all rows of
weights (dequantized one row at a time, fp64 dot products in k order)."""
import os

import numpy as np
import pytest
import torch

import oracle
import w4a16_bit_matmul_amd as wq
import workloads
from parity import FLOOR_GEMV, FLOOR_MFMA, assert_quantize_matches, compare_y, say, to_dev_f16, to_dev_weights

pytestmark = pytest.mark.gpu

_cache = {}


def _quantized(wl):
    """GPU quantization of a workload's weights, checked bit-exact once per
    weight matrix (the sweep's four batch sizes share one)."""
    key = (wl.w_seed, wl.N, wl.K, wl.group, wl.w_dtype)
    if key not in _cache:
        _cache.clear()
        say(f"  generating and quantizing {wl.N}x{wl.K} g={wl.group} ({wl.w_dtype})")
        W = wl.weights()
        oracle.set_threads(min(16, len(os.sched_getaffinity(0))))
        out = wq.wq_quantize_groups(to_dev_weights(W, wl.w_dtype), wl.group, codes=True, packed=True)
        torch.cuda.synchronize()
        q, s, z, _ = assert_quantize_matches(W, wl.w_dtype, wl.group, out=out)
        out.pop("q_codes")
        _cache[key] = (q, s, z, out)
    return _cache[key]


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_workload_full_size(name):
    wl = workloads.WORKLOADS[name]
    say(f"full-size {name}: M={wl.M} N={wl.N} K={wl.K} g={wl.group}")
    q, s, z, out = _quantized(wl)
    x = wl.activations()
    ws_bytes = wq.wq_gemm_workspace_bytes(wl.M, wl.N, wl.K, wl.group)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
    y = wq.wq_gemm_w4a16(to_dev_f16(x), out["qw"], workspace=ws)
    torch.cuda.synchronize()
    floor = FLOOR_MFMA if wq.auto_uses_mfma(wl.M, wl.N, "int4", wl.K, wl.group) else FLOOR_GEMV
    ref = oracle.gemm_rows_f64(x, q, s, z, wl.group, 0, wl.N)
    nw, ew = compare_y(y, ref, floor_frac=floor)
    say(f"  all {wl.M}x{wl.N} outputs: normwise {nw:.2e} elementwise {ew:.2e}")
    if ws is not None:  # the counters are left zero and the workspace reusable: same result again
        assert int(ws[:wq.WQ_WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0
        y2 = wq.wq_gemm_w4a16(to_dev_f16(x), out["qw"], workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)


def test_mlp_up_forced_mfma_full_size():
    """The M=16 up-projection (N=28672, K=8192, g=128) on the MFMA GEMM kernel
    (the default kernel choice runs the split-K GEMV there): every output
    against the oracle."""
    wl = workloads.WORKLOADS["mlp_up_decode"]
    say(f"full-size forced MFMA {wl.name}: M={wl.M} N={wl.N} K={wl.K} g={wl.group}")
    q, s, z, out = _quantized(wl)
    x = wl.activations()
    ws_bytes = wq.wq_gemm_workspace_bytes(wl.M, wl.N, wl.K, wl.group, path=wq.WQ_PATH_MFMA)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
    say(f"  {wq.wq_gemm_plan(wl.M, wl.N, wl.K, wl.group, wq.WQ_PATH_MFMA)}")
    y = wq.wq_gemm_w4a16(to_dev_f16(x), out["qw"], workspace=ws, path=wq.WQ_PATH_MFMA)
    torch.cuda.synchronize()
    ref = oracle.gemm_rows_f64(x, q, s, z, wl.group, 0, wl.N)
    nw, ew = compare_y(y, ref, floor_frac=FLOOR_MFMA)
    say(f"  all {wl.M}x{wl.N} outputs: normwise {nw:.2e} elementwise {ew:.2e}")
