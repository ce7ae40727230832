"""NVFP4 weights on the HIP path against the oracle: the per-tensor scale,
the E4M3 block-scale bytes, the codes and the tile layout bit-exact, decoding
bit-exact, the product within the tolerance on small shapes and at the decode
and M=128 full sizes (every output), one-hot activations selecting decoded
weights exactly.  Every kernel path takes exact operands here (E2M1 times an
E4M3 scale is exact in fp16 and in fp32), so all paths are held to the GEMV's
elementwise floor."""
import os

import numpy as np
import pytest
import torch

import oracle
import w4a16_bit_matmul_amd as wq
import workloads
from parity import FLOOR_GEMV, compare_y, f16_bits, oracle_dtype, say, to_dev_f16, to_dev_weights

pytestmark = pytest.mark.gpu

SHAPES = [(256, 1024), (37, 96), (1000, 1152), (130, 544), (16, 128), (1, 32)]


def gpu_quantize_nv(W_host, w_dtype):
    out = wq.wq_quantize_nvfp4(to_dev_weights(W_host, w_dtype), codes=True)
    torch.cuda.synchronize()
    return out


def assert_nv_matches(W_host, w_dtype, out=None):
    if out is None:
        out = gpu_quantize_nv(W_host, w_dtype)
    q, s8, S = oracle.quantize_nvfp4(W_host, dtype=oracle_dtype(w_dtype))
    S_gpu = float(out["qw"].tensor_scale.cpu().numpy()[0])
    assert S_gpu == S, (S_gpu, S)
    s8_gpu = out["qw"].s8.cpu().numpy()
    assert np.array_equal(s8_gpu, s8), f"scale bytes differ at {np.argwhere(s8_gpu != s8)[:5]}"
    q_gpu = out["q_codes"].cpu().numpy()
    assert np.array_equal(q_gpu, q), f"codes differ at {np.argwhere(q_gpu != q)[:5]}"
    assert np.array_equal(out["qw"].qpacked.cpu().numpy(), oracle.pack_device_mxfp4(q))
    return q, s8, S, out


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("w_dtype", ["f32", "bf16", "f16"])
def test_quantize_nvfp4_bit_exact(N, K, w_dtype):
    say(f"quantize nvfp4 N={N} K={K} {w_dtype}")
    W = workloads.gen_weights(2600 + N + K, N, K, outlier_frac=0.01, dtype="f32")
    if w_dtype == "bf16":
        W = workloads.f32_to_bf16_bits(W)
    elif w_dtype == "f16":
        W = workloads.f32_to_f16_bits(W)
    assert_nv_matches(W, w_dtype)


def test_quantize_nvfp4_special_blocks():
    """A tensor scale that is a power of two (the largest block maps to 448),
    block maxima on E4M3 values and on the midpoints between them (ties to
    even), E2M1 grid points and midpoints inside blocks, all-zero blocks, blocks
    too small for any nonzero scale (codes 0, signs kept) and negative values
    rounding to zero."""
    say("quantize nvfp4 special blocks")
    S = 2.0 ** -10
    e4 = oracle.dequant_nvfp4(np.full((127, 16), 2, np.uint8), np.arange(127, dtype=np.uint8).reshape(-1, 1),
                              1.0)[:, 0].astype(np.float64)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    rows = []
    r = np.zeros(256, np.float32)
    r[0] = 2688 * S  # the tensor maximum: S = 2^-10 exactly
    for b, code in enumerate(range(10, 126, 8)):
        if 1 + b >= 16:
            break
        blk = np.zeros(16)
        d = e4[code] * S
        blk[:8] = grid * d
        blk[8:15] = (grid[:-1] + grid[1:]) / 2 * d
        blk[15] = -0.2 * d
        r[16 * (1 + b):16 * (2 + b)] = blk
    rows.append(r)
    r = np.zeros(256, np.float32)
    for b in range(16):  # block maxima on the midpoints between E4M3 values
        c = 7 * b + 3
        r[16 * b] = (e4[c] + e4[c + 1]) / 2 * 6 * S
        r[16 * b + 1:16 * b + 16] = np.linspace(-1, 1, 15) * r[16 * b]
    rows.append(r)
    rows.append(np.zeros(256, np.float32))
    r = np.zeros(256, np.float32)
    r[:16] = 2.0 ** -9 * 6 * S * 0.24  # rounds to scale 0
    r[16:32] = -r[:16]
    rows.append(r)
    W = np.stack(rows).astype(np.float32)
    q, s8, St, _ = assert_nv_matches(W, "f32")
    assert St == S and np.all(s8[2] == 0) and np.all(q[2] == 0)
    assert s8[3, 0] == 0 and np.all(q[3, :16] == 0) and np.all(q[3, 16:32] == 8)


@pytest.mark.parametrize("N,K", SHAPES)
def test_dequant_nvfp4_bit_exact(N, K):
    say(f"dequant nvfp4 N={N} K={K}")
    rng = np.random.default_rng(N * 5 + K)
    q = rng.integers(0, 16, (N, K)).astype(np.uint8)
    s8 = rng.integers(0, 127, (N, K // 16)).astype(np.uint8)
    s8.flat[0] = 0
    s8.flat[-1] = 126
    S = float(np.float32(rng.uniform(1e-5, 1e-2)))
    qw = wq.QuantizedWeightNV(wq.wq_pack_mxfp4(torch.from_numpy(q).cuda()).qpacked, torch.from_numpy(s8).cuda(),
                              torch.tensor([S], dtype=torch.float32, device="cuda"), N, K)
    torch.cuda.synchronize()
    assert np.array_equal(qw.qpacked.cpu().numpy(), oracle.pack_device_mxfp4(q))
    for td, od in [(torch.float32, oracle.F32), (torch.float16, oracle.F16), (torch.bfloat16, oracle.BF16)]:
        got = wq.wq_dequant_nvfp4(qw, td)
        torch.cuda.synchronize()
        got = got.cpu().numpy() if td == torch.float32 else got.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, oracle.dequant_nvfp4(q, s8, S, od)), td


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
def test_matmul_nvfp4_within_tolerance(M, N, K, path):
    say(f"matmul nvfp4 M={M} N={N} K={K} path={path}")
    seed = 2700 + M + N + K
    W = workloads.gen_weights(seed, N, K, outlier_frac=0.01, dtype="bf16")
    x = workloads.gen_activations(seed + 2, M, K, outlier_frac=0.01)
    out = gpu_quantize_nv(W, "bf16")
    q, s8, S = oracle.quantize_nvfp4(W, dtype=oracle.BF16)
    y_ref = oracle.gemm_rows_nvfp4_f64(x, q, s8, S, 0, N)
    y = wq.wq_gemm_nvfp4(to_dev_f16(x), out["qw"], path=path)
    torch.cuda.synchronize()
    nw, ew = compare_y(y, y_ref, floor_frac=FLOOR_GEMV)
    say(f"  normwise {nw:.2e} elementwise {ew:.2e}")


@pytest.mark.parametrize("path", [wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA])
@pytest.mark.parametrize("M,N,K", [(1, 200, 512), (16, 64, 384), (128, 80, 256), (70, 48, 160)])
def test_nvfp4_one_hot_activations_select_weights_exactly(M, N, K, path):
    """y[m][n] = fp16(fp32(E2M1 * E4M3 * S)) of weight (n, k_m) exactly: the
    oracle's fp16 decoding (one fp32 rounding, then fp16), compared as values."""
    say(f"one-hot nvfp4 M={M} N={N} K={K} path={path}")
    W = workloads.gen_weights(2800 + M, N, K, outlier_frac=0.01, dtype="bf16")
    out = gpu_quantize_nv(W, "bf16")
    q, s8, S = oracle.quantize_nvfp4(W, dtype=oracle.BF16)
    w_hat16 = oracle.dequant_nvfp4(q, s8, S, oracle.F16)
    reps = (min(K, 256) + M - 1) // M
    for rep in range(reps):
        ks = (np.arange(M) + rep * M) % K
        x = np.zeros((M, K), np.float32)
        x[np.arange(M), ks] = 1.0
        y = wq.wq_gemm_nvfp4(to_dev_f16(workloads.f32_to_f16_bits(x)), out["qw"], path=path)
        torch.cuda.synchronize()
        got = f16_bits(y).view(np.float16)
        assert np.array_equal(got, w_hat16[:, ks].T.view(np.float16)), f"rep {rep} columns {ks[:4]}"


@pytest.mark.parametrize("path", [wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA])
@pytest.mark.parametrize("M", [1, 2, 8, 16])
def test_nvfp4_one_hot_every_scale_byte(M, path):
    """Random codes under every E4M3 scale byte 0..126 (the subnormal scales
    m * 2^-9 included), one-hot rows of x: each output is exactly
    fp16(fp32(E2M1 * E4M3 * S)) of one weight, the oracle's decoding."""
    say(f"one-hot nvfp4, every scale byte, M={M} path={path}")
    N, K = 256, 256
    rng = np.random.default_rng(2900 + 10 * M + path)
    q = rng.integers(0, 16, (N, K)).astype(np.uint8)
    s8 = (np.arange(N * K // 16) % 127).astype(np.uint8)
    rng.shuffle(s8)
    s8 = s8.reshape(N, K // 16)
    S = float(np.float32(rng.uniform(0.5, 2.0)))
    qw = wq.QuantizedWeightNV(wq.wq_pack_mxfp4(torch.from_numpy(q).cuda()).qpacked, torch.from_numpy(s8).cuda(),
                              torch.tensor([S], dtype=torch.float32, device="cuda"), N, K)
    w_hat16 = oracle.dequant_nvfp4(q, s8, S, oracle.F16)
    for rep in range(K // M):
        ks = np.arange(M) + rep * M
        x = np.zeros((M, K), np.float32)
        x[np.arange(M), ks] = 1.0
        y = wq.wq_gemm_nvfp4(to_dev_f16(workloads.f32_to_f16_bits(x)), qw, path=path)
        torch.cuda.synchronize()
        got = f16_bits(y).view(np.float16)
        assert np.array_equal(got, w_hat16[:, ks].T.view(np.float16)), f"rep {rep} columns {ks[:4]}"


@pytest.mark.parametrize("name", ["decode_gemv", "batched_gemm"])
def test_nvfp4_workload_full_size(name):
    wl = workloads.WORKLOADS[name]
    say(f"full-size nvfp4 {name}: M={wl.M} N={wl.N} K={wl.K}")
    W = wl.weights()
    oracle.set_threads(min(16, len(os.sched_getaffinity(0))))
    out = wq.wq_quantize_nvfp4(to_dev_weights(W, wl.w_dtype), codes=True)
    torch.cuda.synchronize()
    q, s8, S, _ = assert_nv_matches(W, wl.w_dtype, out=out)
    x = wl.activations()
    ws_bytes = wq.wq_gemm_nvfp4_workspace_bytes(wl.M, wl.N, wl.K)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
    y = wq.wq_gemm_nvfp4(to_dev_f16(x), out["qw"], workspace=ws)
    torch.cuda.synchronize()
    # every output against the oracle's product over all rows of weights
    ref = oracle.gemm_rows_nvfp4_f64(x, q, s8, S, 0, wl.N)
    nw, ew = compare_y(y, ref, floor_frac=FLOOR_GEMV)
    say(f"  all {wl.M}x{wl.N} outputs: normwise {nw:.2e} elementwise {ew:.2e}")
