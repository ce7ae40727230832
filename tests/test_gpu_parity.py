"""HIP path against the oracle, element by element, on seeded inputs small
enough for the oracle to finish in seconds but spanning several tiles, ragged
rows/columns/batch, both groups, all input dtypes and the degenerate cases."""
import numpy as np
import pytest
import torch

import oracle
import w4a16_bit_matmul_amd as wq
import workloads
from parity import (assert_quantize_matches, compare_y, compare_y_path, f16_bits, floor_for, gpu_quantize, ref16, say,
                    split_k, to_dev_f16, to_dev_weights)

pytestmark = pytest.mark.gpu

SHAPES = [  # N, K, group: ragged N (not a multiple of 16 or of any tile), K not a multiple of 128
    (256, 1024, 128),
    (37, 96, 32),
    (1000, 1152, 128),
    (130, 544, 32),
    (16, 128, 128),
    (1, 32, 32),
]


def _weights(N, K, seed, w_dtype="bf16", outliers=0.01):
    return workloads.gen_weights(seed, N, K, outlier_frac=outliers, dtype="f32" if w_dtype == "f32" else "bf16")


# ---------------------------------------------------------------- quantize

@pytest.mark.parametrize("N,K,group", SHAPES)
@pytest.mark.parametrize("w_dtype", ["f32", "bf16"])
def test_quantize_bit_exact(N, K, group, w_dtype):
    say(f"quantize N={N} K={K} g={group} {w_dtype}")
    W = _weights(N, K, 100 + N + K, w_dtype)
    assert_quantize_matches(W, w_dtype, group)


def test_quantize_fp16_input():
    say("quantize fp16 input")
    W = workloads.f32_to_f16_bits(workloads.gen_weights(5, 48, 512, dtype="f32"))
    assert_quantize_matches(W, "f16", 32)


def test_quantize_tiny_workload():
    w = workloads.WORKLOADS["tiny"]
    say(f"quantize {w}")
    assert_quantize_matches(w.weights(), "f32", w.group)


@pytest.mark.parametrize("group", [32, 128])
def test_quantize_worked_example_padded(group):
    """The page's 8 weights padded with zeros to a real group, plus rows built
    to hit the spec's special cases: rounding ties, degenerate groups, groups
    that do not straddle zero, subnormal scales and the stored-scale encode."""
    say(f"quantize special rows g={group}")
    rows = []
    ex = np.zeros(group, np.float32)
    ex[:8] = workloads.WORKED_EXAMPLE_W
    rows.append(ex)
    ties = np.zeros(group, np.float32)
    ties[:8] = [-1.0, 2.75, 0.125, 0.375, -0.875, 2.625, 0.625, -0.125]
    rows.append(ties)
    ztie = np.zeros(group, np.float32)
    ztie[:4] = [-1.125, 2.625, 0.0, 1.0]
    rows.append(ztie)
    rows.append(np.zeros(group, np.float32))
    rows.append(np.full(group, 0.3, np.float32))
    rows.append(np.full(group, -0.3, np.float32))
    rows.append(np.linspace(0.1, 0.5, group).astype(np.float32))
    rows.append(-np.linspace(0.1, 0.5, group).astype(np.float32))
    rows.append(np.full(group, 1e-9, np.float32))
    sub = np.zeros(group, np.float32)
    sub[:4] = [-3e-6, 0.0, 2e-6, 5e-6]
    rows.append(sub)
    s32 = np.float32(3.8) / np.float32(15.0)
    s_h = np.float32(np.float16(s32))
    enc = np.zeros(group, np.float32)
    enc[:3] = [-1.0, 2.8, np.float32(6.5 * (float(s32) + float(s_h)) / 2)]
    rows.append(enc)
    big = np.zeros(group, np.float32)
    big[:2] = [-4.5e5, 4.5e5]  # s = 60000 (near the fp16 limit), -min/s = 7.5 (a tie)
    rows.append(big)
    W = np.stack(rows)
    q, s, z, _ = assert_quantize_matches(W, "f32", group)
    assert list(q[0, :8]) == [8, 5, 11, 6, 15, 0, 7, 10] and z[0, 0] == 6


# ---------------------------------------------------------------- pack / dequant

@pytest.mark.parametrize("N,K,group", SHAPES)
def test_pack_bit_exact(N, K, group):
    say(f"pack N={N} K={K} g={group}")
    rng = np.random.default_rng(N * 7 + K)
    q = rng.integers(0, 16, (N, K)).astype(np.uint8)
    z = rng.integers(0, 16, (N, K // group)).astype(np.uint8)
    qw = wq.wq_pack_int4(torch.from_numpy(q).cuda(), torch.from_numpy(z).cuda(), group)
    torch.cuda.synchronize()
    assert np.array_equal(qw.qpacked.cpu().numpy(), oracle.pack_device(q))
    assert np.array_equal(qw.zpacked.cpu().numpy(), oracle.pack_zeros(z))


@pytest.mark.parametrize("N,K,group", SHAPES)
@pytest.mark.parametrize("out_dtype", ["f32", "f16", "bf16"])
def test_dequant_bit_exact(N, K, group, out_dtype):
    say(f"dequant N={N} K={K} g={group} -> {out_dtype}")
    W = _weights(N, K, 200 + N + K, "f32")
    q, s, z = oracle.quantize_groups(W, group)
    qd = torch.from_numpy(q).cuda()
    zd = torch.from_numpy(z).cuda()
    qw = wq.wq_pack_int4(qd, zd, group)
    qw.s.copy_(torch.from_numpy(s.view(np.int16)).cuda().view(torch.float16))
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out_dtype]
    odt = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16}[out_dtype]
    got = wq.wq_dequant(qw, tdt)
    torch.cuda.synchronize()
    ref = oracle.dequant(q, s, z, group, odt)
    got_np = got.cpu().numpy() if out_dtype == "f32" else got.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got_np.view(np.uint32) if out_dtype == "f32" else got_np,
                          ref.view(np.uint32) if out_dtype == "f32" else ref)


def test_dequant_all_scale_and_code_pairs():
    """Every (q, z) pair under normal, subnormal, tiny and large fp16 scales:
    row i uses scale i; its 16 groups of 32 have zero-points 0..15 and each
    holds the codes 0..15 twice."""
    say("dequant code/zero/scale grid")
    rng = np.random.default_rng(3)
    scales = np.concatenate([np.array([0x0001, 0x03FF, 0x0400, 0x30F8, 0x3C00, 0x7BFF], np.uint16),
                             rng.integers(1, 0x7C00, 26).astype(np.uint16)])
    N, K, group = scales.size, 512, 32
    q = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))
    z = np.tile(np.arange(16, dtype=np.uint8), (N, 1))
    s = np.repeat(scales[:, None], K // group, axis=1)
    qw = wq.wq_pack_int4(torch.from_numpy(q).cuda(), torch.from_numpy(z).cuda(), group)
    qw.s.copy_(torch.from_numpy(s.view(np.int16)).cuda().view(torch.float16))
    for tdt, odt in [(torch.float32, oracle.F32), (torch.float16, oracle.F16), (torch.bfloat16, oracle.BF16)]:
        got = wq.wq_dequant(qw, tdt)
        torch.cuda.synchronize()
        ref = oracle.dequant(q, s, z, group, odt)
        if tdt == torch.float32:
            assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))
        else:
            assert np.array_equal(got.cpu().view(torch.int16).numpy().view(np.uint16), ref)


# ---------------------------------------------------------------- matmul

MATMUL_CASES = [  # M, N, K, group
    (1, 256, 1024, 128),
    (1, 1000, 1152, 128),
    (2, 130, 544, 32),
    (3, 37, 96, 32),
    (5, 300, 512, 32),
    (8, 272, 640, 128),
    (16, 512, 1024, 128),
    (17, 100, 256, 32),
    (33, 160, 384, 128),
    (63, 48, 256, 32),
    (64, 272, 640, 128),
    (77, 130, 1024, 32),
    (128, 512, 2048, 128),
    (130, 100, 256, 128),
    (200, 64, 128, 32),
    # MFMA shapes with a ragged last K tile and partial row tiles: K = 96
    # (one tile, three MFMA steps), 160 (second tile one step), 4224 (33
    # tiles: whole groups of four plus one), 1056 (eight tiles plus one step)
    (40, 100, 96, 32),
    (100, 72, 160, 32),
    (96, 50, 4224, 128),
    (129, 300, 1056, 32),
    # four row blocks per workgroup: 32 to 191 128-column blocks and M > 32
    (40, 4100, 256, 32),
    (100, 4100, 2048, 128),  # and K split two ways
    # eight row blocks per workgroup need at least 192 128-column blocks:
    # N = 24592 gives 193, the last holding a single 16-row block, and M = 130
    # leaves a partial second row tile
    (130, 24592, 384, 32),
    # few row blocks and a K longer than one pass of a workgroup's waves: the
    # GEMV splits K across workgroups
    (1, 48, 28672, 128),
    (2, 1000, 8192, 128),
    (5, 100, 8192, 32),
    (12, 40, 8192, 32),
    # 4-bit GEMV with several 16-row blocks per workgroup (eight or sixteen
    # rows of x): N = 16400 has 1025 row blocks and N = 8200 513, so the last
    # workgroup's later blocks lie past N; M = 30 takes two sixteen-row tiles;
    # N = 8176 (511 blocks), K = 4224: two blocks per workgroup over a ragged
    # K; N = 2064 (129 blocks): one
    (6, 16400, 512, 32),
    (13, 8200, 1024, 128),
    (30, 16400, 512, 32),
    (12, 8176, 4224, 32),
    (16, 2064, 4224, 32),
    # group 32 with K past 16384: AUTO hands M > 8 to the GEMM
    (12, 2064, 16512, 32),
    # eight-row tiles over two blocks: N = 8176 (511 blocks, the last
    # workgroup's second block past N) in sixteen-wave workgroups, and
    # N = 12000 (750 blocks, 375 workgroups) in eight-wave ones
    (8, 8176, 640, 32),
    (6, 12000, 512, 128),
    # narrow outputs with 9..32 rows: eight-row tiles in sixteen-wave
    # workgroups over all of K (no split): one pass with the last row block
    # ragged (N = 1000) and a ragged K (33 tiles), and two passes of the waves
    # over K = 14336 in 260 workgroups
    (24, 1000, 8192, 32),
    (12, 520, 4224, 32),
    (32, 1040, 14336, 128),
]


def _matmul_inputs(M, N, K, group, seed):
    W = workloads.gen_weights(seed, N, K, outlier_frac=0.01, dtype="bf16")
    x = workloads.gen_activations(seed + 2, M, K, outlier_frac=0.01)
    return W, x


@pytest.mark.parametrize("path", [wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA, wq.WQ_PATH_AUTO])
@pytest.mark.parametrize("M,N,K,group", MATMUL_CASES)
def test_matmul_within_tolerance(M, N, K, group, path):
    say(f"matmul M={M} N={N} K={K} g={group} path={path}")
    W, x = _matmul_inputs(M, N, K, group, 300 + M + N + K)
    out = gpu_quantize(W, "bf16", group)
    q, s, z = oracle.quantize_groups(W, group, dtype=oracle.BF16)
    y_ref = oracle.gemm_f64(x, oracle.dequant(q, s, z, group))
    y = wq.wq_gemm_w4a16(to_dev_f16(x), out["qw"], path=path)
    torch.cuda.synchronize()
    nw, ew, ew16 = compare_y_path(y, y_ref, ref16(x, oracle.dequant(q, s, z, group, oracle.F16)), path, M,
                                  K=K, group=group)
    say(f"  normwise {nw:.2e} elementwise {ew:.2e} elementwise vs fp16(What) {ew16}")


@pytest.mark.parametrize("path", [wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA])
@pytest.mark.parametrize("M,N,K,group", [(1, 500, 2048, 128), (3, 300, 1024, 32), (9, 300, 1024, 128),
                                         (64, 200, 1024, 32)])
def test_matmul_offset_activations(M, N, K, group, path):
    """Activations with a common offset (mean 3) and outlier channels (x20):
    each output is then a sum of large terms of both signs (the offset times
    the row's dequantized weights, the outlier channels), and small outputs
    come from their cancellation; checked element by element."""
    say(f"matmul offset activations M={M} N={N} K={K} g={group} path={path}")
    seed = 700 + M + N + K + group
    W = workloads.gen_weights(seed, N, K, outlier_frac=0.01, dtype="bf16")
    x = workloads.gen_activations(seed + 2, M, K, outlier_frac=0.01, outlier_mult=20.0, offset=3.0)
    out = gpu_quantize(W, "bf16", group)
    q, s, z = oracle.quantize_groups(W, group, dtype=oracle.BF16)
    y_ref = oracle.gemm_f64(x, oracle.dequant(q, s, z, group))
    y = wq.wq_gemm_w4a16(to_dev_f16(x), out["qw"], path=path)
    torch.cuda.synchronize()
    nw, ew, ew16 = compare_y_path(y, y_ref, ref16(x, oracle.dequant(q, s, z, group, oracle.F16)), path, M,
                                  K=K, group=group)
    say(f"  normwise {nw:.2e} elementwise {ew:.2e} elementwise vs fp16(What) {ew16}")


@pytest.mark.parametrize("path", [wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA])
@pytest.mark.parametrize("M,N,K,group", [(1, 200, 512, 128), (16, 64, 384, 32), (128, 80, 256, 128),
                                         (70, 48, 160, 32)])
def test_one_hot_activations_select_weights_exactly(M, N, K, group, path):
    """x[m] = e_{k_m}: y[m][n] must be fp16(What[n][k_m]) bit for bit; k_m runs
    over every offset inside a 128-column tile, catching any nibble or lane
    unpacking slip that a norm test could average away."""
    say(f"one-hot M={M} N={N} K={K} g={group} path={path}")
    W = workloads.gen_weights(400 + M, N, K, outlier_frac=0.01, dtype="bf16")
    out = gpu_quantize(W, "bf16", group)
    q, s, z = oracle.quantize_groups(W, group, dtype=oracle.BF16)
    w_hat16 = oracle.dequant(q, s, z, group, oracle.F16)
    reps = (min(K, 256) + M - 1) // M
    for rep in range(reps):
        ks = (np.arange(M) + rep * M) % K
        x = np.zeros((M, K), np.float32)
        x[np.arange(M), ks] = 1.0
        y = wq.wq_gemm_w4a16(to_dev_f16(workloads.f32_to_f16_bits(x)), out["qw"], path=path)
        torch.cuda.synchronize()
        got = f16_bits(y)
        assert np.array_equal(got, w_hat16[:, ks].T), f"rep {rep} columns {ks[:4]}"


@pytest.mark.parametrize("path", [wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA])
def test_grid_exact_weights_reduce_to_fp16_gemm(path):
    """Weights of the form 2^-6 * (c - 7) with every group holding codes 0 and 15
    quantize losslessly, so y is an ordinary fp16 product: compare with the
    fp64 product of the original weights and with torch.matmul."""
    say(f"grid-exact path={path}")
    M, N, K, group = 24, 96, 512, 32
    rng = np.random.default_rng(17)
    c = rng.integers(0, 16, (N, K))
    c[:, ::group] = 0
    c[:, 1::group] = 15
    W = (np.ldexp(1.0, -6) * (c - 7)).astype(np.float32)
    x = workloads.gen_activations(18, M, K)
    out = gpu_quantize(W, "f32", group)
    wh = wq.wq_dequant(out["qw"], torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(wh.cpu(), torch.from_numpy(W))
    y = wq.wq_gemm_w4a16(to_dev_f16(x), out["qw"], path=path)
    torch.cuda.synchronize()
    y_ref = oracle.gemm_f64(x, W)
    compare_y(y, y_ref, floor_frac=floor_for(path, M, N, K=K, group=group))
    y_torch = (to_dev_f16(x).float() @ torch.from_numpy(W).cuda().t()).cpu().numpy().astype(np.float64)
    compare_y(y, y_torch, floor_frac=floor_for(path, M, N, K=K, group=group))


def test_split_k_workspace_is_reusable():
    """Split-K GEMV calls of different shapes share one workspace without
    clearing it in between (each call puts its counters back to zero; the
    partial sums, here pre-filled with NaN bytes, need no clearing), and give
    the same bytes as calls with a fresh zero-filled workspace."""
    say("split-K workspace reuse")
    cases = [(1, 48, 28672, 128), (5, 100, 8192, 32), (2, 1000, 8192, 128), (1, 48, 28672, 128)]
    need = max(wq.wq_gemm_workspace_bytes(M, N, K, g) for M, N, K, g in cases)
    assert need > 0
    shared = torch.zeros(need, dtype=torch.uint8, device="cuda")
    shared[wq.WQ_WORKSPACE_COUNTER_BYTES:] = 0xFF  # partial sums: NaN bytes, never read before written
    for i, (M, N, K, g) in enumerate(cases):
        W, x = _matmul_inputs(M, N, K, g, 600 + i)
        out = gpu_quantize(W, "bf16", g)
        xd = to_dev_f16(x)
        y_shared = wq.wq_gemm_w4a16(xd, out["qw"], workspace=shared, path=wq.WQ_PATH_GEMV)
        fresh = torch.zeros(wq.wq_gemm_workspace_bytes(M, N, K, g), dtype=torch.uint8, device="cuda")
        y_fresh = wq.wq_gemm_w4a16(xd, out["qw"], workspace=fresh, path=wq.WQ_PATH_GEMV)
        torch.cuda.synchronize()
        assert torch.equal(y_shared, y_fresh), (M, N, K, g)
        ctr = wq.WQ_WORKSPACE_COUNTER_BYTES
        assert int(shared[:ctr].count_nonzero()) == 0 and int(fresh[:ctr].count_nonzero()) == 0


def test_mfma_split_k_workspace_is_reusable():
    """MFMA calls whose grid splits K across workgroups (few 128-column blocks)
    share one workspace across shapes without clearing it (partial sums
    pre-filled with NaN bytes), match calls with a fresh zero-filled workspace
    bit for bit, and leave the counters zero."""
    say("MFMA split-K workspace reuse")
    cases = [(8, 256, 8192, 128), (128, 1024, 8192, 32), (70, 300, 4224, 128), (16, 48, 2048, 32), (8, 256, 8192, 128)]
    for M, N, K, g in cases:
        assert split_k(wq.wq_gemm_plan(M, N, K, g, wq.WQ_PATH_MFMA)) > 1, (M, N, K, g)
    need = max(wq.wq_gemm_workspace_bytes(M, N, K, g) for M, N, K, g in cases)
    shared = torch.zeros(need, dtype=torch.uint8, device="cuda")
    shared[wq.WQ_WORKSPACE_COUNTER_BYTES:] = 0xFF  # partial sums: NaN bytes, never read before written
    for i, (M, N, K, g) in enumerate(cases):
        W, x = _matmul_inputs(M, N, K, g, 640 + i)
        out = gpu_quantize(W, "bf16", g)
        xd = to_dev_f16(x)
        y_shared = wq.wq_gemm_w4a16(xd, out["qw"], workspace=shared, path=wq.WQ_PATH_MFMA)
        fresh = torch.zeros(wq.wq_gemm_workspace_bytes(M, N, K, g), dtype=torch.uint8, device="cuda")
        y_fresh = wq.wq_gemm_w4a16(xd, out["qw"], workspace=fresh, path=wq.WQ_PATH_MFMA)
        torch.cuda.synchronize()
        assert torch.equal(y_shared, y_fresh), (M, N, K, g)
        ctr = wq.WQ_WORKSPACE_COUNTER_BYTES
        assert int(shared[:ctr].count_nonzero()) == 0 and int(fresh[:ctr].count_nonzero()) == 0
        q, s, z = oracle.quantize_groups(W, g, dtype=oracle.BF16)
        compare_y(y_shared, oracle.gemm_f64(x, oracle.dequant(q, s, z, g)), floor_frac=floor_for(wq.WQ_PATH_MFMA, M, N))


def test_repeated_calls_are_deterministic():
    say("determinism")
    M, N, K, group = 128, 448, 2048, 128
    W, x = _matmul_inputs(M, N, K, group, 500)
    out = gpu_quantize(W, "bf16", group)
    xd = to_dev_f16(x)
    for path in (wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA):
        y1 = wq.wq_gemm_w4a16(xd, out["qw"], path=path)
        y2 = wq.wq_gemm_w4a16(xd, out["qw"], path=path)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2)
    out2 = gpu_quantize(W, "bf16", group)
    assert torch.equal(out2["qw"].qpacked, out["qw"].qpacked)


@pytest.mark.gpu
def test_sequence_call_matches_single_calls():
    # one host call issuing several products equals the single calls, for the
    # GEMV (with a split-K workspace shared by the sequence) and the MFMA path
    for (M, N, K, group) in [(3, 272, 640, 32), (1, 48, 28672, 128), (80, 100, 512, 128)]:
        say(f"sequence M={M} N={N} K={K} g={group}")
        qws, xs, refs = [], [], []
        for t in range(3):
            W, x = _matmul_inputs(M, N, K, group, 77 + t)
            qw = gpu_quantize(W, "bf16", group)["qw"]
            xd = to_dev_f16(x)
            qws.append(qw)
            xs.append(xd)
            refs.append(wq.wq_gemm_w4a16(xd, qw))
        ys = [torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda") for _ in range(3)]
        wq.wq_gemm_w4a16_seq(xs, qws, ys)
        torch.cuda.synchronize()
        for y, ref in zip(ys, refs):
            assert torch.equal(y, ref)


# ---------------------------------------------------------------- symmetric scheme

@pytest.mark.parametrize("w_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,K,group", SHAPES)
def test_quantize_symmetric_bit_exact(N, K, group, w_dtype):
    say(f"quantize sym N={N} K={K} g={group} {w_dtype}")
    W = _weights(N, K, 900 + N + K, w_dtype)
    q, s, z, _ = assert_quantize_matches(W, w_dtype, group, scheme=wq.WQ_SYM)
    assert np.all(z == 8) and q.min() >= 0 and q.max() <= 15


def test_quantize_symmetric_edge_groups():
    # all-zero groups, exact halves (max |w| = 7: scale 1), one-signed groups,
    # a single outlier, subnormal-scale groups
    say("quantize sym edge groups")
    K, group = 256, 32
    W = np.zeros((16, K), np.float32)
    W[1, :32] = np.array([7.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5] * 4, np.float32)
    W[2, :] = np.abs(np.linspace(0.1, 3.0, K, dtype=np.float32))
    W[3, :] = -np.abs(np.linspace(0.1, 3.0, K, dtype=np.float32))
    W[4, 40] = 30.0
    W[4, 41:64] = np.linspace(-1, 1, 23, dtype=np.float32)
    W[5, :] = np.float32(3e-6) * np.sin(np.arange(K, dtype=np.float32))
    q, s, z, _ = assert_quantize_matches(W, "f32", group, scheme=wq.WQ_SYM)
    assert np.all(q[0] == 8) and np.all(s[0] == 0)
    assert list(q[1, :8].astype(int) - 8) == [7, 0, 2, 2, 0, -2, -2, 4]


@pytest.mark.parametrize("group", [32, 128])
def test_dequant_symmetric_bit_exact(group):
    say(f"dequant sym g={group}")
    N, K = 130, 1152 if group == 128 else 544
    W = workloads.gen_weights(931 + group, N, K, outlier_frac=0.01, dtype="bf16")
    q, s, z, out = assert_quantize_matches(W, "bf16", group, scheme=wq.WQ_SYM)
    got = wq.wq_dequant(out["qw"], torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.dequant(q, s, z, group))


@pytest.mark.parametrize("path", [wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA])
@pytest.mark.parametrize("M,N,K,group", [(1, 1000, 1152, 128), (5, 300, 512, 32), (77, 130, 1024, 32),
                                         (128, 512, 2048, 128), (1, 48, 28672, 128)])
def test_matmul_symmetric_within_tolerance(M, N, K, group, path):
    say(f"matmul sym M={M} N={N} K={K} g={group} path={path}")
    W, x = _matmul_inputs(M, N, K, group, 950 + M + N + K)
    out = gpu_quantize(W, "bf16", group, scheme=wq.WQ_SYM)
    q, s, z = oracle.quantize_groups(W, group, dtype=oracle.BF16, scheme=oracle.SYM)
    y_ref = oracle.gemm_f64(x, oracle.dequant(q, s, z, group))
    y = wq.wq_gemm_w4a16(to_dev_f16(x), out["qw"], path=path)
    torch.cuda.synchronize()
    nw, ew, ew16 = compare_y_path(y, y_ref, ref16(x, oracle.dequant(q, s, z, group, oracle.F16)), path, M,
                                  K=K, group=group)
    say(f"  normwise {nw:.2e} elementwise {ew:.2e} elementwise vs fp16(What) {ew16}")



# ---------------------------------------------------------------- near-tie encodings

def _near_tie_rows(group, rng, lo_mult, hi_mult):
    """Rows whose weights sit on, and a few ulps either side of, the points where
    w / s + z is a half-integer: the first two weights pin the group's range to
    (hi_mult - lo_mult) * s_target with s_target exact in fp16, so the stored
    scale is s_target; the rest are s_target * (k + 1/2), nudged by 0-3 ulps.
    The quantizers' rounding shortcut must agree there with the exact division."""
    rows = []
    for s_target in (1.0, 0.0999755859375, 0.005859375, 7.75, 2.0 ** -20):
        for _ in range(4):
            k = rng.integers(lo_mult, hi_mult, group).astype(np.float32) + np.float32(0.5)
            w = (np.float32(s_target) * k).astype(np.float32)
            for i, d in enumerate(rng.integers(-3, 4, group)):
                for _ in range(abs(int(d))):
                    w[i] = np.nextafter(w[i], np.float32(np.inf if d > 0 else -np.inf))
            w[0], w[1] = np.float32(s_target * hi_mult), np.float32(s_target * lo_mult)
            rows.append(w)
    return np.stack(rows)


@pytest.mark.parametrize("group", [32, 128])
def test_quantize_near_ties_bit_exact(group):
    say(f"near-tie encodings g={group}")
    rng = np.random.default_rng(90 + group)
    assert_quantize_matches(_near_tie_rows(group, rng, -7, 8), "f32", group)
    assert_quantize_matches(_near_tie_rows(group, rng, -7, 7), "f32", group, scheme=wq.WQ_SYM)
    W8 = _near_tie_rows(group, rng, -127, 127)
    out = wq.wq_quantize_w8(to_dev_weights(W8, "f32"), group, codes=True, packed=True)
    torch.cuda.synchronize()
    q, s = oracle.quantize_w8(W8, group)
    assert np.array_equal(out["q_codes"].cpu().numpy(), q) and np.array_equal(f16_bits(out["s"]), s)
    # the same rows as KV-cache blocks of 128
    Wk = _near_tie_rows(128, rng, -7, 8).reshape(-1, 256)
    ref = oracle.kv_alloc(Wk.shape[0], 256)
    oracle.kv_quantize(Wk, ref)
    cache = wq.kv_cache_alloc(Wk.shape[0], 256)
    wq.wq_kv_quantize(torch.from_numpy(Wk).cuda(), cache)
    torch.cuda.synchronize()
    assert np.array_equal(cache.codes.cpu().numpy(), ref[0])
    assert np.array_equal(f16_bits(cache.s), ref[1]) and np.array_equal(cache.zpacked.cpu().numpy(), ref[2])
