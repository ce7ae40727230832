"""AWQ-style per-input-channel scaling on the HIP path against the oracle: the
folded quantization bit-exact, the activation scaling and the channel
statistic bit-exact, and on the decode workload's distribution the fold
lowers the product's error against the unquantized product."""
import numpy as np
import pytest
import torch

import oracle
import w4a16_bit_matmul_amd as wq
import workloads
from parity import FLOOR_GEMV, compare_y, f16_bits, floor_for, say, to_dev_f16, to_dev_weights

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K,group", [(256, 1024, 128), (37, 96, 32), (130, 544, 32)])
@pytest.mark.parametrize("scheme", [wq.WQ_ASYM, wq.WQ_SYM])
def test_quantize_scaled_bit_exact(N, K, group, scheme):
    say(f"quantize scaled N={N} K={K} g={group} scheme={scheme}")
    rng = np.random.default_rng(N + K + scheme)
    W = workloads.gen_weights(700 + N, N, K, outlier_frac=0.01, dtype="bf16")
    alpha = rng.uniform(0.5, 4.0, K).astype(np.float32)
    alpha[rng.choice(K, max(1, K // 100), replace=False)] = 2.0
    out = wq.wq_quantize_groups(to_dev_weights(W, "bf16"), group, codes=True, packed=True, scheme=scheme,
                                alpha=torch.from_numpy(alpha).cuda())
    torch.cuda.synchronize()
    q, s, z = oracle.quantize_groups(W, group, dtype=oracle.BF16, scheme=scheme, alpha=alpha)
    assert np.array_equal(f16_bits(out["s"]), s)
    assert np.array_equal(out["z_codes"].cpu().numpy(), z)
    assert np.array_equal(out["q_codes"].cpu().numpy(), q)
    assert np.array_equal(out["qw"].qpacked.cpu().numpy(), oracle.pack_device(q))
    assert np.array_equal(out["qw"].zpacked.cpu().numpy(), oracle.pack_zeros(z))


@pytest.mark.parametrize("M,K", [(1, 8192), (7, 96), (64, 1024)])
def test_scale_activations_and_statistic_bit_exact(M, K):
    say(f"scale activations / absmean M={M} K={K}")
    rng = np.random.default_rng(M * K)
    x = workloads.gen_activations(800 + M, M, K, outlier_frac=0.01)
    alpha = rng.uniform(0.25, 8.0, K).astype(np.float32)
    xd = to_dev_f16(x)
    got = wq.wq_scale_activations(xd, torch.from_numpy(alpha).cuda())
    stat = wq.wq_channel_absmean(xd)
    torch.cuda.synchronize()
    assert np.array_equal(f16_bits(got), oracle.scale_activations(x, alpha))
    assert np.array_equal(stat.cpu().numpy(), oracle.channel_absmean(x))
    # in place
    wq.wq_scale_activations(xd, torch.from_numpy(alpha).cuda(), out=xd)
    torch.cuda.synchronize()
    assert np.array_equal(f16_bits(xd), oracle.scale_activations(x, alpha))


def _awq_alpha(x_cal, factor, frac=0.01):
    """alpha = factor on the channels with the largest mean |x| over the
    calibration rows (the top `frac` of them), 1 elsewhere -- computed on the
    GPU by the library's statistic; the top-k selection is a host sort."""
    stat = wq.wq_channel_absmean(to_dev_f16(x_cal)).cpu().numpy()
    K = stat.size
    alpha = np.ones(K, np.float32)
    alpha[np.argsort(-stat, kind="stable")[:max(1, int(round(frac * K)))]] = factor
    return alpha


@pytest.mark.parametrize("path", [wq.WQ_PATH_GEMV, wq.WQ_PATH_MFMA])
def test_awq_product_matches_oracle(path):
    say(f"awq product path={path}")
    M, N, K, group = 9, 300, 1024, 128
    W = workloads.gen_weights(901, N, K, outlier_frac=0.001, dtype="bf16")
    x = workloads.gen_activations(902, M, K, outlier_frac=0.01, channel_seed=903)
    x_cal = workloads.gen_activations(904, 64, K, outlier_frac=0.01, channel_seed=903)
    alpha = _awq_alpha(x_cal, 2.0)
    ad = torch.from_numpy(alpha).cuda()
    qw = wq.wq_quantize_groups(to_dev_weights(W, "bf16"), group, alpha=ad)["qw"]
    y = wq.wq_gemm_w4a16(wq.wq_scale_activations(to_dev_f16(x), ad), qw, path=path)
    torch.cuda.synchronize()
    q, s, z = oracle.quantize_groups(W, group, dtype=oracle.BF16, alpha=alpha)
    y_ref = oracle.gemm_f64(oracle.scale_activations(x, alpha), oracle.dequant(q, s, z, group))
    compare_y(y, y_ref, floor_frac=floor_for(path, M, N, K=K, group=group))


def test_awq_fold_reduces_error_on_decode_distribution():
    """The decode workload's weights (8192 x 8192, 0.1 % weight-outlier input
    channels) and activations with 1 % salient channels (x10): folding a factor
    into the salient channels lowers ||y - x W^T|| against the unquantized
    product, for the oracle and for the HIP path alike."""
    wl = workloads.WORKLOADS["decode_gemv"]
    say("awq error reduction, decode distribution")
    W = wl.weights()
    Wd = to_dev_weights(W, "bf16")
    M = 64
    x = workloads.gen_activations(wl.x_seed, M, wl.K, outlier_frac=wl.x_outlier_frac)
    x_cal = workloads.gen_activations(wl.x_seed + 50, 64, wl.K, outlier_frac=wl.x_outlier_frac,
                                      channel_seed=wl.x_seed + 1)
    xd = to_dev_f16(x)
    y_true = (xd.float() @ Wd.float().t()).double()
    plain = wq.wq_quantize_groups(Wd, wl.group)["qw"]
    err_plain = float((wq.wq_gemm_w4a16(xd, plain).double() - y_true).norm())
    errs = {}
    for factor in (1.5, 2.0, 3.0):
        ad = torch.from_numpy(_awq_alpha(x_cal, factor)).cuda()
        qw = wq.wq_quantize_groups(Wd, wl.group, alpha=ad)["qw"]
        y = wq.wq_gemm_w4a16(wq.wq_scale_activations(xd, ad), qw)
        errs[factor] = float((y.double() - y_true).norm())
    torch.cuda.synchronize()
    say(f"  ||y - xW^T||: plain {err_plain:.4f}, folded {errs}")
    assert min(errs.values()) < 0.9 * err_plain
    # the same comparison on the oracle for 32 sampled output columns
    rng = np.random.default_rng(5)
    cols = np.sort(rng.choice(wl.N, 32, replace=False))
    Wc = np.ascontiguousarray(W[cols])
    yt = oracle.gemm_f64(x, workloads.bf16_bits_to_f32(Wc))
    q, s, z = oracle.quantize_groups(Wc, wl.group, dtype=oracle.BF16)
    e_plain = np.linalg.norm(oracle.gemm_f64(x, oracle.dequant(q, s, z, wl.group)) - yt)
    alpha = _awq_alpha(x_cal, 2.0)
    q, s, z = oracle.quantize_groups(Wc, wl.group, dtype=oracle.BF16, alpha=alpha)
    e_fold = np.linalg.norm(oracle.gemm_f64(oracle.scale_activations(x, alpha), oracle.dequant(q, s, z, wl.group)) - yt)
    say(f"  oracle, 32 columns: plain {e_plain:.4f}, folded (x2) {e_fold:.4f}")
    assert e_fold < 0.9 * e_plain
