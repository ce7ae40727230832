"""The allocation-free entry point (wq_gemm_w4a16_noalloc, split-K scratch in
the library's fixed per-GPU array) against wq_gemm_w4a16 with a caller
workspace: bit-identical results on consecutive calls, the first needing the
whole scratch and later ones smaller, and a product needing more scratch than
the array holds rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

import oracle
import w4a16_bit_matmul_amd as wq
import workloads
from parity import compare_y, floor_for, gpu_quantize, say, to_dev_f16

pytestmark = pytest.mark.gpu

# (M, N, K, group): the first needs exactly the scratch's 16 MiB of partial
# sums (MFMA split of the 8192 x 28672 down projection at M = 128); then
# smaller split shapes on the MFMA kernel and on the GEMV, and one that needs
# no scratch at all
CALLS = [(128, 8192, 28672, 32), (8, 1024, 8192, 32), (1, 48, 28672, 128), (1, 8192, 8192, 128)]


def test_noalloc_matches_workspace_entry_point():
    need0 = wq.wq_gemm_workspace_bytes(*CALLS[0], path=wq.WQ_PATH_AUTO)
    assert need0 == wq.WQ_NOALLOC_SCRATCH_BYTES, need0
    for i, (M, N, K, group) in enumerate(CALLS):
        say(f"noalloc call {i}: M={M} N={N} K={K} g={group}: {wq.wq_gemm_plan(M, N, K, group)}")
        W = workloads.gen_weights(6100 + i, N, K, outlier_frac=0.01, dtype="bf16")
        x = workloads.gen_activations(6150 + i, M, K, outlier_frac=0.01)
        qw = gpu_quantize(W, "bf16", group)["qw"]
        xd = to_dev_f16(x)
        need = wq.wq_gemm_workspace_bytes(M, N, K, group, path=wq.WQ_PATH_AUTO)
        assert need <= wq.WQ_NOALLOC_SCRATCH_BYTES
        ws = torch.full((max(need, 1),), 0, dtype=torch.uint8, device="cuda")
        y_ref = wq.wq_gemm_w4a16(xd, qw, workspace=ws)
        y = torch.full_like(y_ref, float("nan"))
        wq.wq_gemm_w4a16_noalloc(xd, qw, y=y)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"call {i}: differs at {(y != y_ref).nonzero()[:4].tolist()}"
        # and within tolerance of the oracle (every output)
        q, s, z = oracle.quantize_groups(W, group, dtype=oracle.BF16)
        nw, ew = compare_y(y, oracle.gemm_rows_f64(x, q, s, z, group, 0, N),
                           floor_frac=floor_for(wq.WQ_PATH_AUTO, M, N, K=K, group=group))
        say(f"  identical to the workspace entry point; normwise {nw:.2e} elementwise {ew:.2e}")
        # the same call again: the scratch's counters were left zero
        y2 = torch.full_like(y_ref, float("nan"))
        wq.wq_gemm_w4a16_noalloc(xd, qw, y=y2)
        torch.cuda.synchronize()
        assert torch.equal(y2, y_ref)


def test_noalloc_rejects_products_beyond_the_scratch():
    # a grid of too few workgroups for the GPU splits K; the first of these
    # shapes whose fp32 partial-sum planes exceed the scratch (384 x 4096 at
    # K = 28672: three splits of 384 x 4096 sums)
    group = 128
    for M, N, K in [(384, 4096, 28672), (128, 12288, 28672), (128, 191 * 128, 20480)]:
        need = wq.wq_gemm_workspace_bytes(M, N, K, group, path=wq.WQ_PATH_AUTO)
        if need > wq.WQ_NOALLOC_SCRATCH_BYTES:
            break
    else:
        pytest.fail("no shape needs more than the scratch")
    # plain device buffers of the right sizes (never read: the call returns first)
    qb, sb, zb = wq.wq_layout_bytes(N, K, group)
    qw = wq.QuantizedWeight(torch.zeros(qb, dtype=torch.uint8, device="cuda"),
                            torch.zeros((N, K // group), dtype=torch.float16, device="cuda"),
                            torch.zeros((N, zb // N), dtype=torch.uint8, device="cuda"), N, K, group)
    x = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(wq.WQError) as err:
        wq.wq_gemm_w4a16_noalloc(x, qw, y=y)
    assert err.value.status == wq.WQ_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())  # nothing ran
