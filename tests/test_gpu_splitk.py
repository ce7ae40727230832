"""The split-K hand-off (fp32 partial sums in a workspace, a per-tile counter,
the last workgroup adds the partials in split order) under repetition, and the
binding's own workspace on a stream other than the current one."""
import numpy as np
import pytest
import torch

import oracle
import w4a16_bit_matmul_amd as wq
import workloads
from parity import FLOOR_GEMV, compare_y, floor_for, gpu_quantize, say, split_k, to_dev_f16

pytestmark = pytest.mark.gpu

# (M, N, K, group, path): shapes whose plan splits K across workgroups, on the
# GEMV (few row blocks, long K) and on the MFMA kernel (few column blocks)
SPLIT_SHAPES = [
    (1, 48, 28672, 128, wq.WQ_PATH_GEMV),
    (2, 1000, 8192, 128, wq.WQ_PATH_GEMV),
    (8, 1024, 8192, 32, wq.WQ_PATH_MFMA),
    (128, 8192, 8192, 128, wq.WQ_PATH_MFMA),
    (128, 8192, 28672, 32, wq.WQ_PATH_MFMA),
]
REPS = 200


def _case(M, N, K, group, seed):
    W = workloads.gen_weights(seed, N, K, outlier_frac=0.01, dtype="bf16")
    x = workloads.gen_activations(seed + 2, M, K, outlier_frac=0.01)
    out = gpu_quantize(W, "bf16", group)
    q, s, z = oracle.quantize_groups(W, group, dtype=oracle.BF16)
    return x, out["qw"], (q, s, z)


def test_split_k_plans_split():
    for M, N, K, group, path in SPLIT_SHAPES:
        plan = wq.wq_gemm_plan(M, N, K, group, path)
        assert split_k(plan) > 1, plan


def test_split_k_repeated_calls_are_identical_and_correct():
    """Every split shape 200 times, the shapes interleaved so that one shared
    workspace's counters pass from shape to shape: each result bit-identical to
    the first call's, the first within tolerance of the oracle over all outputs."""
    cases = []
    need = 0
    for i, (M, N, K, group, path) in enumerate(SPLIT_SHAPES):
        x, qw, qsz = _case(M, N, K, group, 5100 + 17 * i)
        cases.append((M, N, K, group, path, to_dev_f16(x), qw, x, qsz))
        need = max(need, wq.wq_gemm_workspace_bytes(M, N, K, group, path))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    firsts = []
    for M, N, K, group, path, xd, qw, x, (q, s, z) in cases:
        say(f"split-K M={M} N={N} K={K} g={group} path={path}: {wq.wq_gemm_plan(M, N, K, group, path)}")
        y = wq.wq_gemm_w4a16(xd, qw, workspace=ws, path=path)
        torch.cuda.synchronize()
        ref = oracle.gemm_rows_f64(x, q, s, z, group, 0, N)
        nw, ew = compare_y(y, ref, floor_frac=floor_for(path, M, N, K=K, group=group))
        say(f"  normwise {nw:.2e} elementwise {ew:.2e}")
        firsts.append(y.clone())
    outs = [torch.empty_like(f) for f in firsts]
    for rep in range(REPS):
        for (M, N, K, group, path, xd, qw, _, _), y in zip(cases, outs):
            wq.wq_gemm_w4a16(xd, qw, y=y, workspace=ws, path=path)
        torch.cuda.synchronize()
        for c, (f, y) in enumerate(zip(firsts, outs)):
            if not torch.equal(f, y):
                bad = (f != y).nonzero()[:4].tolist()
                pytest.fail(f"repetition {rep}, shape {SPLIT_SHAPES[c]}: differs from the first call at {bad}")
    assert int(ws[:wq.WQ_WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0
    say(f"  {REPS} repetitions of {len(cases)} shapes identical")


@pytest.mark.parametrize("M,N,K,group,path", [SPLIT_SHAPES[0], SPLIT_SHAPES[2]])
def test_split_k_on_a_side_stream_without_workspace(M, N, K, group, path):
    """A split shape on a stream that is not the current one, with no
    workspace passed: the binding's workspace is zero-filled on that stream
    before the product reads its counters."""
    x, qw, _ = _case(M, N, K, group, 5300 + M)
    xd = to_dev_f16(x)
    need = wq.wq_gemm_workspace_bytes(M, N, K, group, path)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    ref = wq.wq_gemm_w4a16(xd, qw, workspace=ws, path=path)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y1 = torch.empty_like(ref)
        y2 = torch.empty_like(ref)
    wq.wq_gemm_w4a16(xd, qw, y=y1, path=path, stream=side)
    wq.wq_gemm_w4a16(xd, qw, y=y2, path=path, stream=side)
    side.synchronize()
    assert torch.equal(y1, ref) and torch.equal(y2, ref)
