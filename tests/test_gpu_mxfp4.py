"""MXFP4 weights on the HIP path against the oracle: codes, E8M0 scale bytes
and the tile layout bit-exact, decoding bit-exact, the product within the
tolerance on small shapes and at the decode and M=128 full sizes (sampled
output columns), one-hot activations selecting decoded weights exactly."""
import os

import numpy as np
import pytest
import torch

import oracle
import w4a16_bit_matmul_amd as wq
import workloads
from parity import (FLOOR_GEMV, FLOOR_MFMA, compare_y, compare_y_path, f16_bits, floor_for, oracle_dtype, ref16, say,
                    to_dev_f16, to_dev_weights)

pytestmark = pytest.mark.gpu

SHAPES = [(256, 1024), (37, 96), (1000, 1152), (130, 544), (16, 128), (1, 32)]


def gpu_quantize_mx(W_host, w_dtype):
    out = wq.wq_quantize_mxfp4(to_dev_weights(W_host, w_dtype), codes=True)
    torch.cuda.synchronize()
    return out


def assert_mx_matches(W_host, w_dtype, out=None):
    if out is None:
        out = gpu_quantize_mx(W_host, w_dtype)
    q, e8 = oracle.quantize_mxfp4(W_host, dtype=oracle_dtype(w_dtype))
    e8_gpu = out["qw"].e8.cpu().numpy()
    assert np.array_equal(e8_gpu, e8), f"scale bytes differ at {np.argwhere(e8_gpu != e8)[:5]}"
    q_gpu = out["q_codes"].cpu().numpy()
    assert np.array_equal(q_gpu, q), f"codes differ at {np.argwhere(q_gpu != q)[:5]}"
    assert np.array_equal(out["qw"].qpacked.cpu().numpy(), oracle.pack_device_mxfp4(q))
    return q, e8, out


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("w_dtype", ["f32", "bf16", "f16"])
def test_quantize_mxfp4_bit_exact(N, K, w_dtype):
    say(f"quantize mxfp4 N={N} K={K} {w_dtype}")
    W = workloads.gen_weights(1600 + N + K, N, K, outlier_frac=0.01, dtype="f32")
    if w_dtype == "bf16":
        W = workloads.f32_to_bf16_bits(W)
    elif w_dtype == "f16":
        W = workloads.f32_to_f16_bits(W)
    assert_mx_matches(W, w_dtype)


def test_quantize_mxfp4_special_blocks():
    """Grid points and midpoints at several block exponents (ties to even),
    saturation past 6, all-zero and fp32-subnormal blocks, negative values
    rounding to zero."""
    say("quantize mxfp4 special blocks")
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    mids = (grid[:-1] + grid[1:]) / 2
    rows = []
    for e in (-20, -3, 0, 7):
        r = np.zeros(128, np.float32)
        r[:8] = grid
        r[8:15] = mids
        r[15:22] = -mids
        r[22] = 7.0
        r[23] = 6.9
        r[24] = -0.2
        r[32:64] = np.linspace(-6, 6, 32)
        r[64:96] = 4.0
        r[96:100] = [7.999, -7.5, 0.25, 0.75]
        rows.append((r * np.float32(2.0 ** e)).astype(np.float32))
    rows.append(np.zeros(128, np.float32))
    rows.append(np.full(128, 1e-40, np.float32))  # fp32 subnormal maximum
    W = np.stack(rows)
    q, e8, _ = assert_mx_matches(W, "f32")
    assert np.all(e8[-2] == 0) and np.all(q[-2] == 0)


@pytest.mark.parametrize("N,K", SHAPES)
def test_pack_and_dequant_mxfp4_bit_exact(N, K):
    say(f"pack / dequant mxfp4 N={N} K={K}")
    rng = np.random.default_rng(N * 3 + K)
    q = rng.integers(0, 16, (N, K)).astype(np.uint8)
    e8 = rng.integers(100, 140, (N, K // 32)).astype(np.uint8)
    e8.flat[0] = 0
    e8.flat[-1] = 252
    qw = wq.wq_pack_mxfp4(torch.from_numpy(q).cuda())
    qw.e8.copy_(torch.from_numpy(e8))
    torch.cuda.synchronize()
    assert np.array_equal(qw.qpacked.cpu().numpy(), oracle.pack_device_mxfp4(q))
    for td, od in [(torch.float32, oracle.F32), (torch.float16, oracle.F16), (torch.bfloat16, oracle.BF16)]:
        got = wq.wq_dequant_mxfp4(qw, td)
        torch.cuda.synchronize()
        got = got.cpu().numpy() if td == torch.float32 else got.cpu().view(torch.int16).numpy().view(np.uint16)
        with np.errstate(over="ignore"):
            assert np.array_equal(got, oracle.dequant_mxfp4(q, e8, od)), td


MATMUL_CASES = [(1, 256, 1024), (1, 1000, 1152), (3, 37, 96), (8, 272, 640), (17, 100, 256), (63, 48, 256),
                (64, 272, 640), (128, 512, 2048), (130, 100, 256), (40, 100, 96), (96, 50, 4224), (129, 300, 1056),
                (1, 48, 28672), (5, 100, 8192),
                # forced GEMV: eight- and sixteen-row tiles over one, two and four
                # row blocks (N past 16384: 1025 blocks, the last one ragged), two rows
                (6, 16400, 512), (16, 16400, 512), (30, 16400, 512), (12, 8176, 4224), (2, 1000, 1152),
                # eight-row tiles over two blocks, sixteen-wave workgroups (511 blocks)
                (8, 8176, 640),
                # narrow outputs, 9..32 rows: eight-row tiles in sixteen-wave
                # workgroups over all of K (one pass, ragged N and K; two passes)
                (24, 1000, 8192), (12, 520, 4224), (32, 1040, 14336)]


@pytest.mark.parametrize("path", [wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA, wq.WQ_PATH_AUTO])
@pytest.mark.parametrize("M,N,K", MATMUL_CASES)
def test_matmul_mxfp4_within_tolerance(M, N, K, path):
    say(f"matmul mxfp4 M={M} N={N} K={K} path={path}")
    seed = 1700 + M + N + K
    W = workloads.gen_weights(seed, N, K, outlier_frac=0.01, dtype="bf16")
    x = workloads.gen_activations(seed + 2, M, K, outlier_frac=0.01)
    out = gpu_quantize_mx(W, "bf16")
    q, e8 = oracle.quantize_mxfp4(W, dtype=oracle.BF16)
    y_ref = oracle.gemm_f64(x, oracle.dequant_mxfp4(q, e8))
    y = wq.wq_gemm_mxfp4(to_dev_f16(x), out["qw"], path=path)
    torch.cuda.synchronize()
    nw, ew, ew16 = compare_y_path(y, y_ref, ref16(x, oracle.dequant_mxfp4(q, e8, oracle.F16)), path, M, fmt="mxfp4")
    say(f"  normwise {nw:.2e} elementwise {ew:.2e} elementwise vs fp16(What) {ew16}")


@pytest.mark.parametrize("path", [wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA])
@pytest.mark.parametrize("M,N,K", [(1, 200, 512), (16, 64, 384), (128, 80, 256), (70, 48, 160)])
def test_mxfp4_one_hot_activations_select_weights_exactly(M, N, K, path):
    """y[m][n] = fp16(What[n][k_m]) exactly, compared as values: a weight of -0
    (a negative value rounded to zero) gives a sum of +0, the sign of a zero
    sum depending on the summation order."""
    say(f"one-hot mxfp4 M={M} N={N} K={K} path={path}")
    W = workloads.gen_weights(1800 + M, N, K, outlier_frac=0.01, dtype="bf16")
    out = gpu_quantize_mx(W, "bf16")
    q, e8 = oracle.quantize_mxfp4(W, dtype=oracle.BF16)
    w_hat16 = oracle.dequant_mxfp4(q, e8, oracle.F16)
    reps = (min(K, 256) + M - 1) // M
    for rep in range(reps):
        ks = (np.arange(M) + rep * M) % K
        x = np.zeros((M, K), np.float32)
        x[np.arange(M), ks] = 1.0
        y = wq.wq_gemm_mxfp4(to_dev_f16(workloads.f32_to_f16_bits(x)), out["qw"], path=path)
        torch.cuda.synchronize()
        got = f16_bits(y).view(np.float16)
        assert np.array_equal(got, w_hat16[:, ks].T.view(np.float16)), f"rep {rep} columns {ks[:4]}"


@pytest.mark.parametrize("name", ["decode_gemv", "batched_gemm"])
def test_mxfp4_workload_full_size(name):
    wl = workloads.WORKLOADS[name]
    say(f"full-size mxfp4 {name}: M={wl.M} N={wl.N} K={wl.K}")
    W = wl.weights()
    oracle.set_threads(min(16, len(os.sched_getaffinity(0))))
    out = wq.wq_quantize_mxfp4(to_dev_weights(W, wl.w_dtype), codes=True)
    torch.cuda.synchronize()
    q, e8, _ = assert_mx_matches(W, wl.w_dtype, out=out)
    x = wl.activations()
    ws_bytes = wq.wq_gemm_mxfp4_workspace_bytes(wl.M, wl.N, wl.K)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
    y = wq.wq_gemm_mxfp4(to_dev_f16(x), out["qw"], workspace=ws)
    torch.cuda.synchronize()
    # every output against the oracle's product over all rows of weights
    floor = FLOOR_MFMA if wq.auto_uses_mfma(wl.M, wl.N, "mxfp4") else FLOOR_GEMV
    ref = oracle.gemm_rows_mxfp4_f64(x, q, e8, 0, wl.N)
    nw, ew = compare_y(y, ref, floor_frac=floor)
    say(f"  all {wl.M}x{wl.N} outputs: normwise {nw:.2e} elementwise {ew:.2e}")
