"""Group absmax int8 weights (W8A16) on the HIP path against the oracle:
quantization, packing and dequantization bit-exact, the product within the
tolerance, on small seeded shapes spanning several tiles with ragged edges and
at the decode and M=128 workloads' full sizes (sampled output columns)."""
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

SHAPES = [(256, 1024, 128), (37, 96, 32), (1000, 1152, 128), (130, 544, 32), (16, 128, 128), (1, 32, 32)]


def gpu_quantize_w8(W_host, w_dtype, group):
    out = wq.wq_quantize_w8(to_dev_weights(W_host, w_dtype), group, codes=True, packed=True)
    torch.cuda.synchronize()
    return out


def assert_w8_matches(W_host, w_dtype, group, out=None):
    """Codes, scales and the tile layout bit-exact against the oracle."""
    if out is None:
        out = gpu_quantize_w8(W_host, w_dtype, group)
    q, s = oracle.quantize_w8(W_host, group, dtype=oracle_dtype(w_dtype))
    s_gpu = f16_bits(out["s"])
    assert np.array_equal(s_gpu, s), f"scales differ at {np.argwhere(s_gpu != s)[:5]}"
    q_gpu = out["q_codes"].cpu().numpy()
    assert np.array_equal(q_gpu, q), f"codes differ at {np.argwhere(q_gpu != q)[:5]}"
    assert np.array_equal(out["qw"].qpacked.cpu().numpy(), oracle.pack_device_w8(q))
    return q, s, out


@pytest.mark.parametrize("N,K,group", SHAPES)
@pytest.mark.parametrize("w_dtype", ["f32", "bf16"])
def test_quantize_w8_bit_exact(N, K, group, w_dtype):
    say(f"quantize w8 N={N} K={K} g={group} {w_dtype}")
    W = workloads.gen_weights(1200 + N + K, N, K, outlier_frac=0.01, dtype="f32" if w_dtype == "f32" else "bf16")
    assert_w8_matches(W, w_dtype, group)


def test_quantize_w8_fp16_input():
    say("quantize w8 fp16 input")
    W = workloads.f32_to_f16_bits(workloads.gen_weights(7, 48, 512, dtype="f32"))
    assert_w8_matches(W, "f16", 128)


@pytest.mark.parametrize("group", [32, 128])
def test_quantize_w8_special_rows(group):
    """The page's four int8 weights (and the same with the outlier 20.0) padded
    to a real group, exact halves at scale 1, an all-zero group, a group whose
    scale underflows fp16, one-signed groups and subnormal scales."""
    say(f"quantize w8 special rows g={group}")
    rows = []
    ex = np.zeros(group, np.float32)
    ex[:4] = [0.12, -0.50, 0.33, 0.90]
    rows.append(ex.copy())
    ex[4] = 20.0
    rows.append(ex)
    ties = np.zeros(group, np.float32)
    ties[:8] = [127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5]
    rows.append(ties)
    rows.append(np.zeros(group, np.float32))
    rows.append(np.full(group, 2.0 ** -40, np.float32))
    rows.append(np.linspace(0.1, 0.5, group).astype(np.float32))
    rows.append(-np.linspace(0.1, 0.5, group).astype(np.float32))
    rows.append((np.float32(1e-4) * np.sin(np.arange(group))).astype(np.float32))
    W = np.stack(rows)
    q, s, _ = assert_w8_matches(W, "f32", group)
    assert list(q[0, :4]) == [17, -71, 47, 127]
    assert list(q[1, :5]) == [1, -3, 2, 6, 127]
    assert list(q[2, :8]) == [127, 0, 2, 2, 0, -2, -2, 126]
    assert np.all(q[3] == 0) and s[3, 0] == 0 and np.all(q[4] == 0) and s[4, 0] == 0


@pytest.mark.parametrize("N,K,group", SHAPES)
def test_pack_int8_bit_exact(N, K, group):
    say(f"pack w8 N={N} K={K}")
    rng = np.random.default_rng(N * 7 + K)
    q = rng.integers(-127, 128, (N, K)).astype(np.int8)
    qw = wq.wq_pack_int8(torch.from_numpy(q).cuda(), group)
    torch.cuda.synchronize()
    assert np.array_equal(qw.qpacked.cpu().numpy(), oracle.pack_device_w8(q))


@pytest.mark.parametrize("N,K,group", SHAPES)
@pytest.mark.parametrize("out_dtype", ["f32", "f16", "bf16"])
def test_dequant_w8_bit_exact(N, K, group, out_dtype):
    say(f"dequant w8 N={N} K={K} g={group} -> {out_dtype}")
    W = workloads.gen_weights(1300 + N + K, N, K, outlier_frac=0.01, dtype="bf16")
    q, s, out = assert_w8_matches(W, "bf16", group)
    td = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out_dtype]
    od = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16}[out_dtype]
    got = wq.wq_dequant_w8(out["qw"], td)
    torch.cuda.synchronize()
    ref = oracle.dequant_w8(q, s, group, od)
    got = got.cpu().numpy() if out_dtype == "f32" else got.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_dequant_w8_all_codes_and_scales():
    """Every code -127..127 under normal, subnormal and extreme fp16 scales,
    through wq_pack_int8 and the standalone dequantization."""
    say("dequant w8 all codes")
    rng = np.random.default_rng(31)
    scales = np.concatenate([np.array([0x0001, 0x0155, 0x03FF, 0x0400, 0x1F42, 0x3C00, 0x7BFF], np.uint16),
                             rng.integers(0x0001, 0x7C00, 25).astype(np.uint16)])
    N, K, group = scales.size, 256, 32
    q = np.zeros((N, K), np.int8)
    q[:, :255] = np.arange(-127, 128, dtype=np.int8)
    s = np.repeat(scales[:, None], K // group, axis=1)
    qw = wq.wq_pack_int8(torch.from_numpy(q).cuda(), group)
    qw.s.copy_(torch.from_numpy(s.view(np.int16)).cuda().view(torch.float16))
    for td, od in [(torch.float32, oracle.F32), (torch.float16, oracle.F16), (torch.bfloat16, oracle.BF16)]:
        got = wq.wq_dequant_w8(qw, td)
        torch.cuda.synchronize()
        got = got.cpu().numpy() if td == torch.float32 else got.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, oracle.dequant_w8(q, s, group, od)), td


MATMUL_CASES = [(1, 256, 1024, 128), (1, 1000, 1152, 128), (3, 37, 96, 32), (8, 272, 640, 128),
                (17, 100, 256, 32), (63, 48, 256, 32), (64, 272, 640, 128), (128, 512, 2048, 128),
                (130, 100, 256, 128), (40, 100, 96, 32), (96, 50, 4224, 128), (129, 300, 1056, 32),
                (1, 48, 8192, 128), (5, 100, 8192, 32),
                # forced GEMV: sixteen-row tiles (one and two of them, ragged N),
                # two rows, and a split K at g = 32
                (16, 2064, 512, 32), (30, 8176, 4224, 128), (12, 8176, 1024, 32), (2, 1000, 1152, 32),
                (1, 48, 28672, 32)]


@pytest.mark.parametrize("path", [wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA, wq.WQ_PATH_AUTO])
@pytest.mark.parametrize("M,N,K,group", MATMUL_CASES)
def test_matmul_w8_within_tolerance(M, N, K, group, path):
    say(f"matmul w8 M={M} N={N} K={K} g={group} path={path}")
    seed = 1400 + M + N + K
    W = workloads.gen_weights(seed, N, K, outlier_frac=0.01, dtype="bf16")
    x = workloads.gen_activations(seed + 2, M, K, outlier_frac=0.01)
    out = gpu_quantize_w8(W, "bf16", group)
    q, s = oracle.quantize_w8(W, group, dtype=oracle.BF16)
    y_ref = oracle.gemm_f64(x, oracle.dequant_w8(q, s, group))
    y = wq.wq_gemm_w8a16(to_dev_f16(x), out["qw"], path=path)
    torch.cuda.synchronize()
    nw, ew, ew16 = compare_y_path(y, y_ref, ref16(x, oracle.dequant_w8(q, s, group, oracle.F16)), path, M, fmt="int8")
    say(f"  normwise {nw:.2e} elementwise {ew:.2e} elementwise vs fp16(What) {ew16}")


@pytest.mark.parametrize("path", [wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA])
@pytest.mark.parametrize("M,N,K,group", [(1, 200, 512, 128), (16, 64, 384, 32), (128, 80, 256, 128),
                                         (70, 48, 160, 32)])
def test_w8_one_hot_activations_select_weights_exactly(M, N, K, group, path):
    """x[m] = e_{k_m} gives y[m][n] = fp16(s * q) bit for bit; k_m covers every
    column offset of a tile, so a byte-order or half-tile slip shows."""
    say(f"one-hot w8 M={M} N={N} K={K} g={group} path={path}")
    W = workloads.gen_weights(1500 + M, N, K, outlier_frac=0.01, dtype="bf16")
    out = gpu_quantize_w8(W, "bf16", group)
    q, s = oracle.quantize_w8(W, group, dtype=oracle.BF16)
    w_hat16 = oracle.dequant_w8(q, s, group, oracle.F16)
    reps = (min(K, 256) + M - 1) // M
    for rep in range(reps):
        ks = (np.arange(M) + rep * M) % K
        x = np.zeros((M, K), np.float32)
        x[np.arange(M), ks] = 1.0
        y = wq.wq_gemm_w8a16(to_dev_f16(workloads.f32_to_f16_bits(x)), out["qw"], path=path)
        torch.cuda.synchronize()
        assert np.array_equal(f16_bits(y), w_hat16[:, ks].T), f"rep {rep} columns {ks[:4]}"


@pytest.mark.parametrize("path", [wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA])
def test_w8_grid_exact_weights_reduce_to_fp16_gemm(path):
    """Weights 2^-9 * c (c in -127..127, every group holding c = 127 or -127)
    quantize losslessly: the product is an ordinary fp16 GEMM."""
    say(f"grid-exact w8 path={path}")
    M, N, K, group = 24, 96, 512, 32
    rng = np.random.default_rng(19)
    c = rng.integers(-127, 128, (N, K))
    c[:, ::group] = np.where(rng.integers(0, 2, (N, K // group)) == 1, 127, -127)
    W = (np.ldexp(1.0, -9) * c).astype(np.float32)
    x = workloads.gen_activations(20, M, K)
    out = gpu_quantize_w8(W, "f32", group)
    wh = wq.wq_dequant_w8(out["qw"], torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(wh.cpu(), torch.from_numpy(W))
    y = wq.wq_gemm_w8a16(to_dev_f16(x), out["qw"], path=path)
    torch.cuda.synchronize()
    compare_y(y, oracle.gemm_f64(x, W), floor_frac=floor_for(path, M, N, "int8"))
    y_torch = (to_dev_f16(x).float() @ torch.from_numpy(W).cuda().t()).cpu().numpy().astype(np.float64)
    compare_y(y, y_torch, floor_frac=floor_for(path, M, N, "int8"))


@pytest.mark.parametrize("name", ["decode_gemv", "batched_gemm"])
def test_w8_workload_full_size(name):
    """The decode (M=1, N=K=8192) and batched (M=128, N=28672, K=8192) shapes
    with int8 weights: quantization bit-exact over the whole matrix, the
    product on every output in the default launch configuration."""
    wl = workloads.WORKLOADS[name]
    say(f"full-size w8 {name}: M={wl.M} N={wl.N} K={wl.K} g={wl.group}")
    W = wl.weights()
    oracle.set_threads(min(16, len(os.sched_getaffinity(0))))
    out = wq.wq_quantize_w8(to_dev_weights(W, wl.w_dtype), wl.group, codes=True, packed=True)
    torch.cuda.synchronize()
    q, s, _ = assert_w8_matches(W, wl.w_dtype, wl.group, out=out)
    x = wl.activations()
    ws_bytes = wq.wq_gemm_w8a16_workspace_bytes(wl.M, wl.N, wl.K, wl.group)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None
    y = wq.wq_gemm_w8a16(to_dev_f16(x), out["qw"], workspace=ws)
    torch.cuda.synchronize()
    # every output against the oracle's product over all rows of weights
    floor = FLOOR_MFMA if wq.auto_uses_mfma(wl.M, wl.N, "int8") else FLOOR_GEMV
    ref = oracle.gemm_rows_w8_f64(x, q, s, wl.group, 0, wl.N)
    nw, ew = compare_y(y, ref, floor_frac=floor)
    say(f"  all {wl.M}x{wl.N} outputs: normwise {nw:.2e} elementwise {ew:.2e}")
